// attn_mixed_fwd for short sequences (N <= 256: at most two 128-key chunks),
// such as ViT-shaped batches.
// The same arithmetic per chunk as k_attn_mixed (FP4 QK^T, the
// integer tile references, P on the 2^-11 grid, FP8 PV with each tile's
// reference in its E8M0 scale, FP16 tiles and vertical lines, the same
// operand layouts), without its software pipeline: with one or two chunks a
// workgroup's time is its prologue, so workgroups are small instead.
//   workgroup = (batch, query head, 64 query rows), 4 waves of 16 rows; the
//               head's MXFP4 K and MXFP8 V^T (and their scales) are staged
//               once in LDS (26 KB at head_dim 64), so several workgroups
//               share a CU;
//   work order: workgroups are dispatched round-robin over the 8 XCDs, so
//               linear id w runs on XCD w % 8; the query tiles of one head
//               take ids that agree mod 8 and follow one another on that XCD
//               (head 8 (r / n_t) + w % 8, tile r % n_t with r = w / 8), and
//               the head's K and V leave HBM for one L2 only;
//   FP16 tiles and line keys read their bf16 K rows and fp16 V^T straight
//   from global memory into the MFMA operand registers (bounds-checked
//   buffer loads; unused entries read zeros).
#include "attn_common.h"

namespace mxq {
namespace attn {
namespace {

template <int D, bool LINES>
__global__ void __launch_bounds__(256, 4) k_attn_short(AttnArgs a) {
  using LY = Lds<D>;
  constexpr int BQ = 64;   // query rows per workgroup
  constexpr int NT = 256;  // 4 waves of 16 rows
  constexpr int KROW = D / 2;
  constexpr int NDB = D / 16;
  constexpr int NSB = D / 32;
  constexpr int NCH = 2;   // 128-key chunks
  constexpr float NEG_INF = -__builtin_inff();

  __shared__ __attribute__((aligned(16))) uint8_t s_k[NCH][128 * KROW];  // K codes, Lds<D>::k_off layout
  __shared__ __attribute__((aligned(16))) uint8_t s_v[NCH][D * 128];     // V^T codes, Lds<D>::vrow_off layout
  // scales in their global order: K [key][D/32] of the N keys (then 16
  // padding bytes), V [row d][N/32 key blocks]
  __shared__ __attribute__((aligned(16))) uint8_t s_ks[NCH * 128 * NSB + 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_vs[D * NCH * 4];
  __shared__ uint32_t s_lm[NCH][4];  // line keys of a chunk per lane group: bit 16t + (key & 15)

  const int tid = lane_tid();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int n_t = a.N / BQ;
  const uint32_t wr = wg_x() >> 3;
  const uint32_t wq = mdiv(wr, a.mg_nt);
  const int head = static_cast<int>(wq * 8 + (wg_x() & 7));
  if (head >= a.nbh) return;  // the whole workgroup: grid rounded up to whole groups of 8 heads
  const int it = static_cast<int>(wr - wq * n_t);
  const int b = static_cast<int>(mdiv(head, a.mg_hq)), h = head - b * a.Hq;
  const int64_t bhq = static_cast<int64_t>(b) * a.Hq + h;
  const int64_t bhk = static_cast<int64_t>(b) * a.Hkv + static_cast<int>(mdiv(h, a.mg_g));
  const int qs = it * BQ;
  const int q = qs + wave * 16 + col;

  if (qs >= a.n_valid) {  // a tile of padding rows: output 0, lse -inf
    for (int idx = tid; idx < BQ * D; idx += NT) {
      const int64_t o = (bhq * a.N + qs) * D + idx;
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
  last_tile = __builtin_amdgcn_readfirstlane(last_tile);
  const int n_chunks = (last_tile + 2) / 2;  // 1 or 2
  const float c = a.c;

  auto rsrc = [](const void* base, int64_t off_bytes, int64_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base) + (base ? off_bytes : 0);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
    const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(base ? bytes : 0));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), 0, n,
                                             0x00020000);
  };
  const auto r_qc = rsrc(a.q_codes, bhq * a.N * KROW, static_cast<int64_t>(a.N) * KROW);
  const auto r_qs = rsrc(a.q_scales, bhq * a.N * NSB, static_cast<int64_t>(a.N) * NSB);
  const auto r_kc = rsrc(a.k_codes, bhk * a.N * KROW, static_cast<int64_t>(a.N) * KROW);
  const auto r_ks = rsrc(a.k_scales, bhk * a.N * NSB, static_cast<int64_t>(a.N) * NSB);
  const auto r_vc = rsrc(a.v_codes, bhk * D * a.N, static_cast<int64_t>(D) * a.N);
  const auto r_vs = rsrc(a.v_scales, bhk * D * (a.N / 32), static_cast<int64_t>(D) * (a.N / 32));
  const auto r_hk = rsrc(a.k_bf16, bhk * a.N * D * 2, static_cast<int64_t>(a.N) * D * 2);
  const auto r_hv = rsrc(a.v_f16t, bhk * D * a.N * 2, static_cast<int64_t>(D) * a.N * 2);
  const bool lv_bf16 = a.v_f16t == nullptr;  // line V from bf16 V rows (no FP16 tile is promoted)
  const auto r_lv = lv_bf16 ? rsrc(a.v_bf16, bhk * a.N * D * 2, static_cast<int64_t>(a.N) * D * 2) : r_hv;
  constexpr int kOut = 0x7FFFFFF0;  // an offset past every slice: the load returns zeros
  // the head's line list goes out first: the line rows' loads depend on it
  int line_raw = -1;
  if constexpr (LINES) line_raw = (lane < 16 && lane < a.n_lines) ? a.lines[bhq * a.n_lines + lane] : -1;

  // ---- the FP4 Q fragment (B operand of S^T = K Q^T; groups g >= D/32 read
  // zero codes and a zero scale byte) and the bf16 Q slices of FP16 tiles
  const v4i qw = __builtin_bit_cast(
      v4i, __builtin_amdgcn_raw_buffer_load_b128(r_qc, g < NSB ? q * KROW + 16 * g : kOut, 0, 0));
  const v8i qf4 = {qw[0], qw[1], qw[2], qw[3], 0, 0, 0, 0};
  const int qsc = __builtin_amdgcn_raw_buffer_load_b8(r_qs, g < NSB ? q * NSB + g : kOut, 0, 0);
  v8bf qbr[NSB];
#pragma unroll
  for (int st = 0; st < NSB; ++st) qbr[st] = v8bf{};
  if (a.mode != MXQ_ALL_LOWBIT || LINES) {
#pragma unroll
    for (int st = 0; st < NSB; ++st)
      qbr[st] = *reinterpret_cast<const v8bf*>(a.q_bf16 + bhq * a.N * D + (q * D + 8 * (4 * st + g)));
  }

  // ---- stage the head's low-bit K and V (both chunks) in LDS by direct
  // global-to-LDS copies (64 lanes x 16 B per wave instruction, or 4 B per
  // lane for nothing here): each LDS 16-byte unit p of a chunk's K or V^T
  // buffer is fetched from the global unit its layout assigns to it; chunks
  // past the slice read zeros.  The scales are copied as they lie in memory
  // (the head's K scales and V scales are each one contiguous run of at most
  // 1 KB); lanes read their scale bytes from there.
  const bool lowbit = a.mode != MXQ_ALL_FP16;
  constexpr int KUC = 128 * KROW / 16;  // 16-byte K units per chunk
  constexpr int VUC = D * 8;            // 16-byte V^T units per chunk
  static_assert((NCH * KUC) % (64 * 4) == 0 && (NCH * VUC) % (64 * 4) == 0, "whole wave copies");
  auto lds_dma16 = [](const __amdgpu_buffer_rsrc_t& r, uint8_t* dst, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
  };
  if (lowbit) {
#pragma unroll
    for (int i = 0; i < NCH * KUC / 256; ++i) {  // K: LDS unit p of chunk ch
      const int pu = (i * 4 + wave) * 64 + lane;
      const int ch = pu / KUC, p = pu % KUC;
      int key, gu;
      if constexpr (D == 128) {
        key = p >> 2;
        gu = (p & 3) ^ (2 * ((key >> 5) & 1));
      } else {
        key = LY::k_row(p >> 1);
        gu = p & 1;
      }
      lds_dma16(r_kc, &s_k[0][0] + 1024 * (i * 4 + wave), (ch * 128 + key) * KROW + 16 * gu);
    }
#pragma unroll
    for (int i = 0; i < NCH * VUC / 256; ++i) {  // V^T: LDS unit p = row d, slot u
      const int pu = (i * 4 + wave) * 64 + lane;
      const int ch = pu / VUC, p = pu % VUC;
      const int d = p >> 3, u = (p & 7) ^ ((d >> 1) & 7);
      lds_dma16(r_vc, &s_v[0][0] + 1024 * (i * 4 + wave), d * a.N + ch * 128 + 16 * u);
    }
    const int ksb = a.N * NSB, vsb = D * (a.N / 32);  // scale bytes of the head (multiples of 16)
    if (wave == 0 && 16 * lane < ksb) lds_dma16(r_ks, s_ks, 16 * lane);
    if (wave == 1 && 16 * lane < vsb) lds_dma16(r_vs, s_vs, 16 * lane);
    // padding after the K scales: lane groups g >= D/32 of the last key read
    // here (against zero Q codes); 127 is a finite E8M0
    if (tid < 16) s_ks[ksb + tid] = 127;
  }
  // ---- vertical-line keys (HyQuant): entry e takes part when 0 <= key <
  // n_valid and it exceeds every earlier entry (exclusive prefix maximum by DPP
  // row shifts); lane e < 16 of every wave holds entry e's key, else -1
  int lkey = -1;
  if constexpr (LINES) {
    const int raw = line_raw;
    constexpr int kMin = -2147483647 - 1;
    int v = raw;
    v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x111, 0xF, 0xF, false));  // row_shr:1
    v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x112, 0xF, 0xF, false));  // row_shr:2
    v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x114, 0xF, 0xF, false));  // row_shr:4
    v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x118, 0xF, 0xF, false));  // row_shr:8
    const int before = __builtin_amdgcn_update_dpp(kMin, v, 0x111, 0xF, 0xF, false);
    if (lane < 16 && raw >= 0 && raw < a.n_valid && raw > before) lkey = raw;
  }
  // entry e's key, from lane e (an LDS permute: the copies in flight are
  // counted on the vector-memory counter, not the LDS one)
  auto lane_key = [&](int e) -> int { return __shfl(lkey, e); };
  // the line tile's operands, loaded before the barrier so that their round
  // trip overlaps the staging: entry col's bf16 K row (A of the bf16 MFMA)
  // and the fp16 V of entries 4g..4g+3 for rows 16*db + col; entry slot i is
  // loaded only where some lane group has a counted entry there (a list of
  // one line loads one slot)
  v8bf lka[NSB];
  int lk4[4] = {-1, -1, -1, -1};
  v4h vl[NDB];
  if constexpr (LINES) {
    const int kcol_key = lane_key(col);
#pragma unroll
    for (int st = 0; st < NSB; ++st)
      lka[st] = __builtin_bit_cast(
          v8bf, __builtin_amdgcn_raw_buffer_load_b128(r_hk, kcol_key >= 0 ? (kcol_key * D + 32 * st + 8 * g) * 2
                                                                            : kOut, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) lk4[i] = lane_key(4 * g + i);
    const uint32_t used = static_cast<uint32_t>(__ballot(lane < 16 && lkey >= 0));
#pragma unroll
    for (int db = 0; db < NDB; ++db) vl[db] = v4h{};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!(used & (0x1111u << i))) continue;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int off = lv_bf16 ? (lk4[i] * D + 16 * db + col) * 2 : ((16 * db + col) * a.N + lk4[i]) * 2;
        const uint32_t hv = __builtin_amdgcn_raw_buffer_load_b16(r_lv, lk4[i] >= 0 ? off : kOut, 0, 0);
        vl[db][i] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(line_v_f16(hv, lv_bf16)));
      }
    }
  }
  // word (chunk, lane group) of the line-key bits: wave 0 clears the words
  // and its lanes 0..15 OR in their entries' bits (one wave's LDS operations
  // complete in order, so the clears land first)
  if (wave == 0) {
    if (lane < NCH * 4) (&s_lm[0][0])[lane] = 0u;
    if constexpr (LINES) {
      if (lkey >= 0)  // a counted entry lies below n_valid <= N <= 256
        __hip_atomic_fetch_or(&s_lm[lkey >> 7][(lkey >> 4) & 3], 1u << (16 * ((lkey >> 6) & 1) + (lkey & 15)),
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __syncthreads();  // staged codes, scales and line bits

  v4f O[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) O[i] = v4f{0.f, 0.f, 0.f, 0.f};
  v4f L = {0.f, 0.f, 0.f, 0.f};
  float m_run = NEG_INF;  // running integer reference (log2 units)
  float m_o = NEG_INF;    // reference O and L are expressed in
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

  if constexpr (LINES) {
    // the line tile, first in the reference order: S^T[16 entries x 16 queries]
    // with the bf16 MFMA (entry col's K row as A), P = fp16(2^x), then V^T of
    // the entries (fp16, [d][entry]) times P^T with the 16x16x16 fp16 MFMA
    v4f SL = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NSB; ++st) SL = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lka[st], qbr[st], SL, 0, 0, 0);
    float mx = NEG_INF;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = lk4[i] >= 0 && q < a.n_valid && (!a.causal || lk4[i] <= q);
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
    for (int db = 0; db < NDB; ++db) O[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(vl[db], ph, O[db], 0, 0, 0);
    const v4h ones4 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f),
                       static_cast<_Float16>(1.0f)};
    L = __builtin_amdgcn_mfma_f32_16x16x16f16(ones4, ph, L, 0, 0, 0);
  }

  // promotion flags of this workgroup's rows (one selection row: 64 rows lie
  // in one 64- or 128-row selection tile)
  const uint32_t* mrow = (a.mode == MXQ_MIXED && a.mask)
                             ? a.mask + (bhq * (a.N >> a.sel_shift) + (qs >> a.sel_shift)) * a.words
                             : nullptr;
  constexpr int kOne8 = 0x38383838, kOne16 = 0x3C003C00;
  const v8i ones8 = {kOne8, kOne8, kOne8, kOne8, kOne8, kOne8, kOne8, kOne8};
  const int kbase0 = LY::k_off(chunk_key(0, col), g);
  const int kbase1 = LY::k_off(chunk_key(1, col), g);
  auto koff = [&](int beta) -> int {
    if constexpr (D == 128) {
      return kbase0 + LY::KROW * (64 * (beta >> 2) + 4 * (beta & 3));
    } else {
      return (beta & 1 ? kbase1 : kbase0) + LY::KROW * (64 * (beta >> 2) + 4 * (beta & 2));
    }
  };
  const int voff = LY::vrow_off(col, g);

  // a wave whose 16 rows are all padding computes nothing (its rows are
  // written as zeros); in other waves padding rows need no mask: their Q is
  // zero, so their scores are finite, and their output is replaced by zeros
  const int n_ch_wave = __builtin_amdgcn_readfirstlane(qs + 16 * wave) < a.n_valid ? n_chunks : 0;
  // keys a row may see: below n_valid, and up to the row itself when causal
  const int kmax = a.causal ? min(a.n_valid, q + 1) : a.n_valid;
#pragma unroll 1
  for (int ch = 0; ch < n_ch_wave; ++ch) {
    const int kc = ch * 128;
    const bool valid1 = 2 * ch + 1 <= last_tile;
    v4f S[8];
    if (lowbit) {
      // K scale byte of (key ch*128 + chunk_key(beta, col), block g), one
      // register per MFMA (op_sel 0)
      const uint8_t* ksb = &s_ks[(ch * 128 + chunk_key(0, col)) * NSB + g];
#pragma unroll
      for (int beta = 0; beta < 8; ++beta) {
        const v4i w = *reinterpret_cast<const v4i*>(&s_k[ch][koff(beta)]);
        const v8i ka = {w[0], w[1], w[2], w[3], 0, 0, 0, 0};
        const int sc = ksb[NSB * (64 * (beta >> 2) + 4 * (beta & 3))];
        S[beta] = MXQ_QK_BLOCK(0);
      }
    } else {
#pragma unroll
      for (int beta = 0; beta < 8; ++beta) S[beta] = v4f{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
    }
    int fl = 0;  // bit t: tile t of the chunk is FP16 for these rows
    if (a.mode == MXQ_ALL_FP16) {
      fl = 1 | (valid1 ? 2 : 0);
    } else if (a.mode == MXQ_MIXED) {
      const uint32_t w = mrow[(2 * ch) >> 5];
      fl = static_cast<int>((w >> ((2 * ch) & 31)) & 1u) |
           (valid1 ? static_cast<int>(((w >> ((2 * ch + 1) & 31)) & 1u) << 1) : 0);
    }
    float m_tile0 = NEG_INF;
    float low0 = NEG_INF, low1 = NEG_INF;  // row maxima of the low-bit scores left in each tile
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t == 1 && !valid1) {
#pragma unroll
        for (int bb = 4; bb < 8; ++bb) S[bb] = v4f{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
        break;
      }
      const bool prom = (fl >> t) & 1;
      const int kt0 = kc + 64 * t;
      v4f St[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) St[bb] = S[4 * t + bb];
      if (prom) {  // bf16 QK^T of the tile, K rows straight from global memory
#pragma unroll
        for (int st = 0; st < NSB; ++st) {
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const int key = 16 * (col >> 2) + 4 * bb + (col & 3);
            const v8bf ka = __builtin_bit_cast(
                v8bf, __builtin_amdgcn_raw_buffer_load_b128(r_hk, ((kt0 + key) * D + 32 * st + 8 * g) * 2, 0, 0));
            St[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qbr[st], st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : St[bb],
                                                             0, 0, 0);
          }
        }
      }
      // this lane's 16 keys kt0 + 16g + j, j = 4bb + i, are visible for j below
      // nvis (kmax) and when not a line key (bit j of lm); the scores are
      // rewritten only in tiles where some lane has a hidden key
      const int nvis = min(max(kmax - (kt0 + 16 * g), 0), 16);
      if (__any(nvis < 16)) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * bb + i >= nvis) St[bb][i] = NEG_INF;
      }
      if constexpr (LINES) {
        const uint32_t lm = (s_lm[ch][g] >> (16 * t)) & 0xFFFFu;
        if (__any(lm != 0u)) {
#pragma unroll
          for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if ((lm >> (4 * bb + i)) & 1u) St[bb][i] = NEG_INF;
        }
      }
      float mx = NEG_INF;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) mx = fmaxf(fmaxf(mx, fmaxf(St[bb][0], St[bb][1])), fmaxf(St[bb][2], St[bb][3]));
      mx = rowmax4(mx);
      const float m_t = fmaxf(m_run, ceilf(mx * c));
      m_run = m_t;
      if (t == 0) m_tile0 = m_t;
      if (prom) {
        // P relative to O's reference m_o <= m_t (exact scaling while fp16 is
        // normal); O is rebased when 2^(m_t - m_o) would leave fp16's range
        if (m_o == NEG_INF) m_o = m_t;
        else if (__any(m_t - m_o > kMaxLag16)) rebase(m_t);
        const float m_ref = m_o == NEG_INF ? 0.0f : m_o;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          v8h ph;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            ph[e] = static_cast<_Float16>(__builtin_amdgcn_exp2f(__builtin_fmaf(St[2 * st + (e >> 2)][e & 3], c, -m_ref)));
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const v8h va = __builtin_bit_cast(
                v8h, __builtin_amdgcn_raw_buffer_load_b128(r_hv, ((16 * db + col) * a.N + kt0 + 16 * g + 8 * st) * 2,
                                                           0, 0));
            O[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ph, O[db], 0, 0, 0);
          }
          const v8h ones16 = __builtin_bit_cast(v8h, v4i{kOne16, kOne16, kOne16, kOne16});
          L = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones16, ph, L, 0, 0, 0);
        }
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) St[bb] = v4f{NEG_INF, NEG_INF, NEG_INF, NEG_INF};  // no low-bit P
      } else {
        if (t == 0) low0 = mx;
        else low1 = mx;
      }
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) S[4 * t + bb] = St[bb];
    }
    // ---- low-bit P and PV of the chunk; each tile's reference enters through
    // the E8M0 scale of its P blocks, 2^-8 * 2^(m_t - m_o)
    const float hm0 = m_tile0, hm1 = m_run;
    auto live = [&](float rmax, float href) -> bool {
      const float off = kGridMagic + kExpOffset - (href == NEG_INF ? 0.0f : href);
      return __any(__builtin_fmaf(rmax, c, off) > kGridMagic - 10.0f);
    };
    if (live(low0, hm0) || live(low1, hm1)) {
      if (m_o == NEG_INF) m_o = m_run;
      else if (__any(m_run - m_o > kMaxLag)) rebase(m_run);
      const float off0 = kGridMagic + kExpOffset - (hm0 == NEG_INF ? 0.0f : hm0);
      const float off1 = kGridMagic + kExpOffset - (hm1 == NEG_INF ? 0.0f : hm1);
      v8i pb;
#pragma unroll
      for (int beta = 0; beta < 8; ++beta) pb[beta] = p4_e4m3(S[beta], c, beta < 4 ? off0 : off1);
      const float mt = g < 2 ? hm0 : hm1;
      const int psc = (mt == NEG_INF || m_o == NEG_INF)
                          ? 0 : static_cast<int>(fminf(fmaxf(static_cast<float>(kPScale) + (mt - m_o), 0.0f), 254.0f));
      // V scale byte of (row 16*db + col, key block 4*ch + g)
      const uint8_t* vsb = &s_vs[col * (a.N / 32) + 4 * ch + g];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const v4i w0 = *reinterpret_cast<const v4i*>(&s_v[ch][2048 * db + voff]);
        const v4i w1 = *reinterpret_cast<const v4i*>(&s_v[ch][2048 * db + (voff ^ 64)]);
        const v8i va = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
        const int vs = vsb[16 * db * (a.N / 32)];
        O[db] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, pb, O[db], 0, 0, 0, vs, 0, psc);
      }
      L = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones8, pb, L, 0, 0, 0, 127, 0, psc);
    }
  }

  // ---------------------------------------------------------------- epilogue
  const bool row_ok = q < a.n_valid;
  const float l = L[0];
  const float inv = row_ok ? 1.0f / l : 0.0f;
  // the head's rows from a scalar base and a 32-bit row offset, formed here
  // (the row index is made opaque, so no per-lane 64-bit address from the
  // prologue stays live across the kernel)
  int qo = q;
  __asm__ volatile("" : "+v"(qo));
  const int64_t obase = bhq * a.N * D;
  const int orow = qo * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d0 = 16 * db + 4 * g;
    const float o0 = O[db][0] * inv, o1 = O[db][1] * inv, o2 = O[db][2] * inv, o3 = O[db][3] * inv;
    if (a.out_bf16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + obase + (orow + d0)) =
          make_uint2(bf16x2_rne(o0, o1), bf16x2_rne(o2, o3));
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + obase + (orow + d0)) = make_float4(o0, o1, o2, o3);
    }
  }
  if (a.lse && g == 0) a.lse[bhq * a.N + qo] = row_ok ? (m_o + __log2f(l)) * 0.69314718055994531f : NEG_INF;
}

template <int D>
mxq_status launch_short_d(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((a.nbh + 7) / 8 * 8 * (a.N / 64)));
  if (a.n_lines > 0) hipLaunchKernelGGL((k_attn_short<D, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_attn_short<D, false>), grid, dim3(256), 0, st, a);
  return check_launch("k_attn_short");
}

}  // namespace

mxq_status launch_short(const AttnArgs& a, int D, hipStream_t st) {
  return D == 128 ? launch_short_d<128>(a, st) : launch_short_d<64>(a, st);
}

}  // namespace attn
}  // namespace mxq

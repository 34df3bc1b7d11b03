// attn_select_blocks: stage 1 of ThriftAttention (abstract) -- a cheap
// heuristic picks the query-key tiles that run in FP16; HyQuant (abstract)
// adds the sink column and the local window as always-high-precision tiles.
//
// Two kernels:
//  k_tile_means : fp32 mean of every query tile (per query head) and key tile
//                 (per kv head); one thread per (tile, d), rows summed in
//                 ascending order, then one correctly rounded division.
//  k_select     : one workgroup per (b, query head, up to 8 query tiles):
//                 scores of all key tiles against each tile mean (sequential
//                 over d, rounded product then rounded sum, never fused) -- or
//                 of the group's shared tile mean (R35), or the max-pooled key
//                 logits (R37) --, forced tiles, and the top-k by a radix
//                 search for the k-th largest score with ties to the lower
//                 index.
// The fixed operation order makes the result bit-identical to a plain CPU
// evaluation of the same formula.
#include <algorithm>

#include "mxq_internal.h"

// Every product and sum in this file is rounded on its own, as written: with
// contraction off the compiler may not fuse a*b+c into one FMA.  (HIP's
// __fmul_rn/__fadd_rn are plain * and + defined in a header, so they would
// still be fused; plain operators under this pragma are not.)
#pragma clang fp contract(off)

namespace mxq {
namespace {

constexpr int kMaxKeyTiles = 2048;

// mean of rows [tile*T, tile*T + T) of x (capped at n_valid), column d.  The
// row loads are issued 64 at a time; the sum is taken in ascending row order.
// transposed == 0 writes mean[(bh*n_tiles + tile)*D + d], else
// mean[(bh*D + d)*n_tiles + tile] (so that a thread per key tile reads a
// column of means with consecutive threads at consecutive addresses).
__global__ void __launch_bounds__(128) k_tile_means(const uint16_t* __restrict__ x, float* __restrict__ mean,
                                                    int N, int D, int T, int n_valid, int n_tiles,
                                                    int transposed) {
  const int d = threadIdx.x;
  const int tile = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (d >= D) return;
  const uint16_t* base = x + (bh * N + static_cast<int64_t>(tile) * T) * D + d;
  const int rows = max(0, min(T, n_valid - tile * T));
  float acc = 0.0f;
  int r = 0;
  for (; r + 64 <= rows; r += 64) {
    uint16_t v[64];
#pragma unroll
    for (int u = 0; u < 64; ++u) v[u] = base[static_cast<int64_t>(r + u) * D];
#pragma unroll
    for (int u = 0; u < 64; ++u) acc = acc + bf16_to_f32(v[u]);
    __builtin_amdgcn_sched_barrier(0);  // 64 loads in flight at a time
  }
  for (; r < rows; ++r) acc = acc + bf16_to_f32(base[static_cast<int64_t>(r) * D]);
  const float m = rows > 0 ? acc / static_cast<float>(rows) : 0.0f;  // correctly rounded division
  if (transposed) mean[(bh * D + d) * n_tiles + tile] = m;
  else mean[(bh * n_tiles + tile) * D + d] = m;
}

struct SelectArgs {
  const float* qmean;  // [B*Hq][n_qt][D]
  const float* kmean;  // [B*Hkv][D][n_kt] (transposed)
  uint32_t* mask;      // [B*Hq][n_qt][words]
  int32_t* n_fp16;     // [B*Hq][n_qt] or null
  float* scores;       // [B*Hq][n_qt][n_kt] or null
  int Hq, Hkv, N, n_valid, D, Bq, Bk, causal, n_qt, n_kt, words;
  int topk, ratio_num, ratio_den, sink_tiles, local_tiles;
  int B;
  int score_free;  // no tile is chosen by score and none is reported: skip the scores
  int shared;      // one mask per kv group: the G heads' tile means averaged (reading R35)
  int maxkey;      // scores from the max-pooled key logits (reading R37); needs k
  const uint16_t* k;  // bf16 [B*Hkv][N][D] (maxkey only)
  int qt;          // query tiles per workgroup
};

// Workgroup = (batch, query head, qt consecutive query tiles), four waves:
//  1. the qt tile means (or the kv group's shared means) go to LDS as [d][row];
//  2. scores of every key tile.  Tile-mean heuristic: thread t takes key tiles
//     t, t + 256, ... and accumulates the qt dot products side by side, d
//     ascending (each still a sequential sum of rounded products), so a key
//     tile's mean column is read once for all qt rows.  Max-pooled key logits:
//     wave w takes rows w, w + 4, ..., a lane per key;
//  3. wave w selects rows w, w + 4, ...: forced tiles, the k best candidates
//     by a radix search over order-preserving keys of the scores (forced and
//     invalid tiles key 0), and one ballot per 64 tiles for the mask words.
// D (64 or 128) is a compile-time constant so that a column's loads go out 32
// at a time before their products.  Scores live in dynamic LDS, [row][stride]
// with stride = n_kt rounded up to 64.
constexpr int kSelWaves = 4;
constexpr int kSelMaxQT = 8;          // query tiles per workgroup
constexpr int kSelLdsBytes = 32768;   // the score rows' LDS

template <int D>
__global__ void __launch_bounds__(64 * kSelWaves) k_select(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) float s_dyn[];  // [qt][stride] scores, then keys
  __shared__ __attribute__((aligned(16))) float s_q[D][kSelMaxQT];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int qt = a.qt;
  const int nblk = (a.n_qt + qt - 1) / qt;
  const int64_t bhq = static_cast<int64_t>(blockIdx.x) / nblk;  // b * Hq + h
  const int i0 = static_cast<int>(static_cast<int64_t>(blockIdx.x) % nblk) * qt;
  const int nrows = min(qt, a.n_qt - i0);
  const int h = static_cast<int>(bhq % a.Hq);
  const int64_t bhk = (bhq / a.Hq) * a.Hkv + h / (a.Hq / a.Hkv);
  const int stride = (a.n_kt + 63) & ~63;

  if (!a.score_free) {
    for (int idx = tid; idx < D * kSelMaxQT; idx += 64 * kSelWaves) {
      const int r = idx / D, d = idx % D;
      float v = 0.0f;
      if (r < nrows) {
        const int i = i0 + r;
        if (a.shared) {
          // the kv group's shared tile mean: the G heads' means summed in head
          // order, one division by G (every head of the group computes the same)
          const int G = a.Hq / a.Hkv;
          const int64_t bh0 = bhq - h % G;
          float acc = 0.0f;
          for (int hh = 0; hh < G; ++hh) acc = acc + a.qmean[((bh0 + hh) * a.n_qt + i) * D + d];
          v = acc / static_cast<float>(G);
        } else {
          v = a.qmean[(bhq * a.n_qt + i) * D + d];
        }
      }
      s_q[d][r] = v;
    }
    __syncthreads();

    if (a.maxkey) {
      // max-pooled key logits: for each key tile, lane l takes key 64 j + l,
      // its dot product with the tile mean (d ascending, rounded products and
      // sums), and the wave's maximum is the tile's score (-inf when no key of
      // the tile is valid).  Only the row's valid tiles unless every score is
      // reported.
      const uint16_t* kb = a.k + bhk * a.N * D;
      for (int r = wave; r < nrows; r += kSelWaves) {
        const int i = i0 + r;
        float* sc = s_dyn + r * stride;
        int jmax = a.n_kt;
        if (!a.scores) {
          const int qs = i * a.Bq;
          if (qs >= a.n_valid) {
            jmax = 0;
          } else {
            const int qe = min(qs + a.Bq, a.n_valid) - 1;
            int last = (a.n_valid - 1) / a.Bk;
            if (a.causal) last = min(last, qe / a.Bk);
            jmax = last + 1;
          }
        }
        for (int j = 0; j < jmax; ++j) {
          const int key = j * a.Bk + lane;
          float acc = -__builtin_inff();
          if (key < a.n_valid) {
            const uint4* row = reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(key) * D);
            acc = 0.0f;
#pragma unroll 4
            for (int u = 0; u < D / 8; ++u) {
              const uint4 w = row[u];
              const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t bits = (e & 1) ? (ww[e >> 1] & 0xFFFF0000u) : (ww[e >> 1] << 16);
                acc = acc + s_q[8 * u + e][r] * __uint_as_float(bits);  // two roundings: contraction is off
              }
            }
          }
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) acc = fmaxf(acc, __shfl_xor(acc, off));
          if (lane == 0) {
            sc[j] = acc;
            if (a.scores) a.scores[(bhq * a.n_qt + i) * a.n_kt + j] = acc;
          }
        }
      }
    } else {
      // kmean[bhk] ([D][n_kt]) as a buffer: thread offset plus a scalar row offset
      const uint64_t km_base = reinterpret_cast<uint64_t>(a.kmean + bhk * D * a.n_kt);
      const uint32_t km_lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(km_base));
      const uint32_t km_hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(km_base >> 32));
      const auto r_km = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<void*>((static_cast<uint64_t>(km_hi) << 32) | km_lo), 0,
          __builtin_amdgcn_readfirstlane(D * a.n_kt * 4), 0x00020000);
      // scores of every key tile (also invalid ones, for inspection)
      for (int j = tid; j < a.n_kt; j += 64 * kSelWaves) {
        // the tile means are re-read from LDS for every key tile: kept in
        // registers across iterations they would spill
        __asm__ volatile("" ::: "memory");
        float acc[kSelMaxQT];
#pragma unroll
        for (int r = 0; r < kSelMaxQT; ++r) acc[r] = 0.0f;
        constexpr int C = 32;  // loads in flight per round trip
#pragma unroll
        for (int d0 = 0; d0 < D; d0 += C) {
          float kv[C];
#pragma unroll
          for (int d = 0; d < C; ++d)
            kv[d] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_km, 4 * j, 4 * (d0 + d) * a.n_kt, 0));
#pragma unroll
          for (int d = 0; d < C; ++d) {
            const float4 q0 = *reinterpret_cast<const float4*>(&s_q[d0 + d][0]);
            const float4 q1 = *reinterpret_cast<const float4*>(&s_q[d0 + d][4]);
            const float qv[kSelMaxQT] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
            for (int r = 0; r < kSelMaxQT; ++r) acc[r] = acc[r] + qv[r] * kv[d];  // two roundings: contraction is off
            // a few means in registers at a time: the sums so far are pinned
            // here and later LDS reads stay below (compiler-only fences; the
            // optimiser would otherwise hoist every read to the top)
            if (d % 4 == 3) {
#pragma unroll
              for (int r = 0; r < kSelMaxQT; ++r) __asm__ volatile("" : "+v"(acc[r]));
              __asm__ volatile("" ::: "memory");
            }
          }
          __asm__ volatile("" ::: "memory");  // the next chunk's loads stay behind (register budget)
        }
#pragma unroll
        for (int r = 0; r < kSelMaxQT; ++r) {
          if (r < nrows) {
            s_dyn[r * stride + j] = acc[r];
            if (a.scores) a.scores[(bhq * a.n_qt + i0 + r) * a.n_kt + j] = acc[r];
          }
        }
      }
    }
  }  // (score_free: the budget below is 0, so no score is ever read)
  __syncthreads();

  for (int r = wave; r < nrows; r += kSelWaves) {
    const int i = i0 + r;
    float* sc = s_dyn + r * stride;
    uint32_t* mrow = a.mask + (bhq * a.n_qt + i) * a.words;
    const int qs = i * a.Bq;
    int count = 0;
    if (qs < a.n_valid) {
      const int qe = min(qs + a.Bq, a.n_valid) - 1;
      int last = (a.n_valid - 1) / a.Bk;
      if (a.causal) last = min(last, qe / a.Bk);
      const int nvt = last + 1;
      const int lo = qs - (a.local_tiles - 1) * a.Bk;
      auto forced = [&](int j) {
        bool sink = j < a.sink_tiles;
        bool local = a.local_tiles >= 1 && (j + 1) * a.Bk - 1 >= lo && j * a.Bk <= qe;
        return sink || local;
      };
      // forced tiles: the sink tiles [0, ns) and the window tiles [lw, hw]
      const int ns = min(a.sink_tiles, nvt);
      int n_forced = ns;
      if (a.local_tiles >= 1) {
        const int lw = max(0, (lo >= 0 ? lo : lo - a.Bk + 1) / a.Bk), hw = min(nvt - 1, qe / a.Bk);
        if (hw >= lw) n_forced += (hw - lw + 1) - max(0, min(hw, ns - 1) - lw + 1);
      }
      const int n_cand = nvt - n_forced;
      int64_t k;
      if (a.topk >= 0) k = a.topk;
      else k = (static_cast<int64_t>(a.ratio_num) * nvt + a.ratio_den - 1) / a.ratio_den;
      if (k > n_cand) k = n_cand;
      // The k best candidates by (score descending, index ascending), found as
      // the k-th largest score by a radix search over order-preserving keys:
      // a candidate's score becomes an unsigned key that orders as the float
      // does (-0 first made +0, the two compare equal), a forced or invalid tile
      // key 0, below every candidate (a finite score's key is at least
      // 0x00800000).  Each of the 32 passes fixes one bit of the k-th largest
      // key by counting, with ballots, the keys that match the bits fixed so
      // far and have this bit set.
      uint32_t* key = reinterpret_cast<uint32_t*>(sc);
      const int nm = (nvt + 63) / 64;  // 64-tile groups holding valid tiles
      for (int j = lane; j < nm * 64; j += 64) {
        uint32_t u = 0u;
        if (j < nvt && !forced(j)) {
          const uint32_t bits = __float_as_uint(sc[j] + 0.0f);  // -0 -> +0
          u = bits ^ ((bits >> 31) ? 0xFFFFFFFFu : 0x80000000u);
        }
        key[j] = u;
      }
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      uint32_t thr = 0u;  // the k-th largest key (valid when 0 < k < n_cand)
      int k_eq = 0;       // how many keys equal to thr are taken (lowest indices first)
      if (k > 0 && k < n_cand) {
        uint32_t hi_mask = 0u;
        int need = static_cast<int>(k);
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t b = 1u << bit;
          int cnt = 0;
          for (int m = 0; m < nm; ++m) {
            const uint32_t u = key[64 * m + lane];
            cnt += __popcll(__ballot((u & hi_mask) == thr && (u & b) != 0u));
          }
          if (cnt >= need) thr |= b;
          else need -= cnt;
          hi_mask |= b;
        }
        k_eq = need;
      }
      int eq_before = 0;  // keys equal to thr at lower indices, over the groups done
      for (int j0 = 0; j0 < a.n_kt; j0 += 64) {
        const int j = j0 + lane;
        bool take = j < nvt && forced(j);
        if (j < nvt && !take && k > 0) {
          const uint32_t u = key[j];
          if (k >= n_cand) {
            take = true;
          } else {
            const bool eq = u == thr;
            const uint64_t eqb = __ballot(eq);
            const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(eqb >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(eqb), 0));
            take = u > thr || (eq && eq_before + below < k_eq);
          }
        }
        // equal keys of this group (all lanes take part in the ballot)
        if (k > 0 && k < n_cand)
          eq_before += __popcll(__ballot(j < nvt && key[j < nm * 64 ? j : 0] == thr && j < nm * 64));
        const uint64_t bits = __ballot(take);
        count += __popcll(bits);
        if (lane < 2 && j0 / 32 + lane < a.words) mrow[j0 / 32 + lane] = static_cast<uint32_t>(bits >> (32 * lane));
      }
    } else {
      for (int w = lane; w < a.words; w += 64) mrow[w] = 0u;
    }
    if (lane == 0 && a.n_fp16) a.n_fp16[bhq * a.n_qt + i] = count;
  }
}

// ---- vertical-line tokens (HyQuant, summary and abstract: single key
// positions that queries all along the sequence attend to stay in full
// precision).  Probe of a head: the mean of its valid query tiles' means (of
// the G heads of its kv group when lines are shared), summed tile by tile in
// ascending order and divided once; score of key j: probe . k_j, fp32, d
// ascending, rounded product then rounded sum.
constexpr int kMaxLines = 16;

// line lists made of the first n_first keys only: entry e = e, then -1
__global__ void __launch_bounds__(256) k_lines_first(int32_t* __restrict__ lines, int total, int n_lines,
                                                     int n_first) {
  const int idx = static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x);
  if (idx >= total) return;
  const int e = idx % n_lines;
  lines[idx] = e < n_first ? e : -1;
}

struct LineArgs {
  const float* qmean;   // [B*Hq][n_qt][D]
  const uint16_t* k;    // bf16 [B*Hkv][N][D]
  float* ws_scores;     // [B*Hsel][N]
  float* scores;        // [B*Hq][N] or null
  int32_t* lines;       // [B*Hq][n_lines]
  int Hq, Hkv, N, n_valid, D, n_qt, n_vt, shared, n_lines, sink;
};

// One thread per key; every workgroup rebuilds the probe of its head (a few
// hundred adds per head_dim element).
__global__ void __launch_bounds__(256) k_line_scores(LineArgs a) {
  __shared__ float s_probe[256];
  const int hs = blockIdx.y, b = blockIdx.z;  // hs: query head, or kv head when shared
  const int G = a.Hq / a.Hkv;
  const int nh = a.shared ? G : 1;
  const int h0 = a.shared ? hs * G : hs;
  const int hk = a.shared ? hs : hs / G;
  const int Hsel = a.shared ? a.Hkv : a.Hq;
  for (int d = threadIdx.x; d < a.D; d += blockDim.x) {
    float acc = 0.0f;
    for (int h = 0; h < nh; ++h) {
      const float* qm = a.qmean + (static_cast<int64_t>(b) * a.Hq + h0 + h) * a.n_qt * a.D + d;
      for (int i = 0; i < a.n_vt; ++i) acc = acc + qm[static_cast<int64_t>(i) * a.D];
    }
    s_probe[d] = acc / static_cast<float>(nh * a.n_vt);
  }
  __syncthreads();
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= a.N) return;
  float v = -__builtin_inff();
  if (j < a.n_valid) {
    const uint4* row = reinterpret_cast<const uint4*>(a.k + ((static_cast<int64_t>(b) * a.Hkv + hk) * a.N + j) * a.D);
    float acc = 0.0f;
    for (int u = 0; u < a.D / 8; ++u) {
      const uint4 w = row[u];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (e & 1) ? (ww[e >> 1] & 0xFFFF0000u) : (ww[e >> 1] << 16);
        acc = acc + __uint_as_float(bits) * s_probe[8 * u + e];  // two roundings: contraction is off
      }
    }
    v = acc;
  }
  a.ws_scores[(static_cast<int64_t>(b) * Hsel + hs) * a.N + j] = v;
  if (a.scores)
    for (int h = 0; h < nh; ++h) a.scores[(static_cast<int64_t>(b) * a.Hq + h0 + h) * a.N + j] = v;
}

// (v, j) ranks before (w, i): higher score, or the same score and lower index
__device__ __forceinline__ bool line_before(float v, int j, float w, int i) {
  return v > w || (v == w && j < i);
}

// One workgroup per (b, head or kv group): every thread keeps the best 16
// candidates of its keys (j = tid + 256 m) in registers, sorted; the workgroup
// then takes the overall best n_lines - sinks by repeated argmax over the
// threads' list heads (ties to the lower index, as the key order defines).
__global__ void __launch_bounds__(256) k_line_topk(LineArgs a) {
  constexpr int T = 256;
  __shared__ float s_v[T / 64];
  __shared__ int s_j[T / 64];
  __shared__ int s_take[kMaxLines];
  const int hs = blockIdx.x, b = blockIdx.y;
  const int G = a.Hq / a.Hkv;
  const int Hsel = a.shared ? a.Hkv : a.Hq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sink = min(min(a.sink, a.n_valid), a.n_lines);
  const int k = min(a.n_lines - sink, a.n_valid - sink);
  const float* sc = a.ws_scores + (static_cast<int64_t>(b) * Hsel + hs) * a.N;
  float lv[kMaxLines];
  int lj[kMaxLines];
#pragma unroll
  for (int e = 0; e < kMaxLines; ++e) { lv[e] = -__builtin_inff(); lj[e] = 0x7FFFFFFF; }
  for (int j = sink + tid; j < a.n_valid; j += T) {
    float v = sc[j];
    int jj = j;
    // insertion into the sorted list: bubble the new entry up from the tail
#pragma unroll
    for (int e = 0; e < kMaxLines; ++e) {
      if (line_before(v, jj, lv[e], lj[e])) {
        const float tv = lv[e];
        const int tj = lj[e];
        lv[e] = v; lj[e] = jj;
        v = tv; jj = tj;
      }
    }
  }
  int head = 0;  // this thread's first unused list entry
  for (int r = 0; r < k; ++r) {
    float v = -__builtin_inff();
    int j = 0x7FFFFFFF;
#pragma unroll
    for (int e = 0; e < kMaxLines; ++e)
      if (e == head) { v = lv[e]; j = lj[e]; }
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(v, off);
      const int oj = __shfl_xor(j, off);
      if (line_before(ov, oj, v, j)) { v = ov; j = oj; }
    }
    if (lane == 0) { s_v[wave] = v; s_j[wave] = j; }
    __syncthreads();
    float bv = s_v[0];
    int bj = s_j[0];
    for (int w = 1; w < T / 64; ++w)
      if (line_before(s_v[w], s_j[w], bv, bj)) { bv = s_v[w]; bj = s_j[w]; }
    __syncthreads();
    // keys are distinct, so exactly one thread's head holds the winner
    if (bj < a.n_valid && (bj - sink) % T == tid) ++head;
    if (tid == 0) s_take[r] = bj;
  }
  __syncthreads();
  if (tid == 0) {
    int out[kMaxLines];
    int n = 0;
    for (int e = 0; e < sink; ++e) out[n++] = e;
    for (int r = 0; r < k; ++r) {  // insertion sort of the chosen keys (all >= sink)
      int key = s_take[r], p = n;
      while (p > sink && out[p - 1] > key) { out[p] = out[p - 1]; --p; }
      out[p] = key;
      ++n;
    }
    const int nh = a.shared ? G : 1;
    const int h0 = a.shared ? hs * G : hs;
    for (int h = 0; h < nh; ++h) {
      int32_t* dst = a.lines + (static_cast<int64_t>(b) * a.Hq + h0 + h) * a.n_lines;
      for (int e = 0; e < a.n_lines; ++e) dst[e] = e < n ? out[e] : -1;
    }
  }
}

mxq_status validate_shape(const mxq_attn_shape* s) {
  MXQ_REQUIRE(s != nullptr, MXQ_EINVAL, "shape is NULL");
  MXQ_REQUIRE(s->B >= 1 && s->Hq >= 1 && s->Hkv >= 1 && s->N >= 1, MXQ_EINVAL,
              "shape: B, Hq, Hkv, N must be >= 1");
  MXQ_REQUIRE(s->Hq % s->Hkv == 0, MXQ_EINVAL, "shape: Hq must be a multiple of Hkv");
  MXQ_REQUIRE(s->n_valid >= 1 && s->n_valid <= s->N, MXQ_EINVAL, "shape: n_valid must be in [1, N]");
  MXQ_REQUIRE(s->D == 64 || s->D == 128, MXQ_EUNSUPPORTED, "shape: D must be 64 or 128");
  MXQ_REQUIRE(s->Bk == 64, MXQ_EUNSUPPORTED, "shape: Bk must be 64");
  MXQ_REQUIRE(s->Bq == 64 || s->Bq == 128, MXQ_EUNSUPPORTED, "shape: Bq must be 64 or 128");
  MXQ_REQUIRE(s->N % 128 == 0, MXQ_EUNSUPPORTED, "shape: N must be a multiple of 128");
  MXQ_REQUIRE(s->N / s->Bk <= kMaxKeyTiles, MXQ_EUNSUPPORTED, "shape: at most 2048 key tiles");
  MXQ_REQUIRE(s->B <= 65535 && s->Hq <= 65535, MXQ_EUNSUPPORTED, "shape: B and Hq must be <= 65535");
  MXQ_REQUIRE(s->causal == 0 || s->causal == 1, MXQ_EINVAL, "shape: causal must be 0 or 1");
  return MXQ_OK;
}

}  // namespace

mxq_status validate_attn_shape(const mxq_attn_shape* s) { return validate_shape(s); }

}  // namespace mxq

using namespace mxq;

extern "C" size_t attn_select_blocks_workspace(const mxq_attn_shape* s) {
  if (s == nullptr || s->Bq <= 0 || s->Bk <= 0) return 0;
  size_t n_qt = static_cast<size_t>(s->N / s->Bq), n_kt = static_cast<size_t>(s->N / s->Bk);
  return (static_cast<size_t>(s->B) * s->Hq * n_qt + static_cast<size_t>(s->B) * s->Hkv * n_kt) *
         static_cast<size_t>(s->D) * sizeof(float);
}

// k_select over given tile means (layouts as k_tile_means writes them)
static mxq_status launch_select(const float* qmean, const float* kmean, const uint16_t* k_bf16,
                                const mxq_attn_shape* s,
                                const mxq_select_params* p, uint32_t* mask, int32_t* n_fp16, float* scores,
                                bool score_free, hipStream_t strm) {
  const int n_qt = s->N / s->Bq, n_kt = s->N / s->Bk;
  SelectArgs a;
  a.qmean = qmean; a.kmean = kmean; a.mask = mask; a.n_fp16 = n_fp16; a.scores = scores;
  a.Hq = s->Hq; a.Hkv = s->Hkv; a.N = s->N; a.n_valid = s->n_valid; a.D = s->D; a.Bq = s->Bq;
  a.Bk = s->Bk; a.causal = s->causal; a.n_qt = n_qt; a.n_kt = n_kt; a.words = (n_kt + 31) / 32;
  a.topk = p->topk; a.ratio_num = p->ratio_num; a.ratio_den = p->ratio_den;
  a.sink_tiles = p->sink_tiles; a.local_tiles = p->local_tiles;
  a.B = s->B;
  a.score_free = score_free ? 1 : 0;
  a.shared = p->group_shared ? 1 : 0;
  a.maxkey = p->heuristic == 1 ? 1 : 0;
  a.k = k_bf16;
  const int stride = (n_kt + 63) / 64 * 64;
  // up to 8 query tiles share a workgroup (fewer when a score row is wide),
  // and fewer still while the launch would hold under 512 workgroups
  int qt = std::max(1, std::min(kSelMaxQT, kSelLdsBytes / (4 * stride)));
  const int64_t heads = static_cast<int64_t>(s->Hq) * s->B;
  while (qt > 1 && static_cast<int64_t>((n_qt + qt - 1) / qt) * heads < 512) --qt;
  a.qt = qt;
  const int64_t wgs = static_cast<int64_t>((n_qt + a.qt - 1) / a.qt) * s->Hq * s->B;
  MXQ_REQUIRE(wgs <= 0x7FFFFF, MXQ_EUNSUPPORTED, "attn_select_blocks: too many (batch, head, query tile) groups");
  const size_t lds = static_cast<size_t>(a.qt) * stride * sizeof(float);
  const dim3 grid(static_cast<unsigned>(wgs));
  if (s->D == 128) hipLaunchKernelGGL(k_select<128>, grid, dim3(64 * kSelWaves), lds, strm, a);
  else hipLaunchKernelGGL(k_select<64>, grid, dim3(64 * kSelWaves), lds, strm, a);
  return check_launch("k_select");
}

static mxq_status check_select_params(const mxq_select_params* p) {
  MXQ_REQUIRE(p != nullptr, MXQ_EINVAL, "attn_select_blocks: params is NULL");
  MXQ_REQUIRE(p->topk >= 0 || (p->ratio_num >= 0 && p->ratio_den > 0), MXQ_EINVAL,
              "attn_select_blocks: need topk >= 0 or ratio_num >= 0 and ratio_den > 0");
  MXQ_REQUIRE(p->group_shared == 0 || p->group_shared == 1, MXQ_EINVAL,
              "attn_select_blocks: group_shared must be 0 or 1");
  MXQ_REQUIRE(p->heuristic == 0 || p->heuristic == 1, MXQ_EINVAL,
              "attn_select_blocks: heuristic must be 0 (tile means) or 1 (max-pooled key logits)");
  MXQ_REQUIRE(p->sink_tiles >= 0 && p->local_tiles >= 0, MXQ_EINVAL,
              "attn_select_blocks: sink_tiles and local_tiles must be >= 0");
  return MXQ_OK;
}

extern "C" mxq_status attn_select_blocks_means(const float* q_means, const float* k_means,
                                               const mxq_attn_shape* s, const mxq_select_params* p,
                                               uint32_t* mask, int32_t* n_fp16, float* scores,
                                               mxq_stream_t stream) {
  mxq_status st = validate_shape(s);
  if (st != MXQ_OK) return st;
  if ((st = check_select_params(p)) != MXQ_OK) return st;
  MXQ_REQUIRE(q_means != nullptr && k_means != nullptr && mask != nullptr, MXQ_EINVAL,
              "attn_select_blocks_means: q_means, k_means and mask are required");
  MXQ_REQUIRE(p->heuristic == 0, MXQ_EUNSUPPORTED,
              "attn_select_blocks_means: the max-pooled key heuristic needs the key rows (attn_select_blocks)");
  return launch_select(q_means, k_means, nullptr, s, p, mask, n_fp16, scores, false, as_stream(stream));
}

extern "C" mxq_status attn_select_blocks(const uint16_t* q, const uint16_t* k,
                                         const mxq_attn_shape* s, const mxq_select_params* p,
                                         void* workspace, size_t ws_bytes, uint32_t* mask,
                                         int32_t* n_fp16, float* scores, mxq_stream_t stream) {
  mxq_status st = validate_shape(s);
  if (st != MXQ_OK) return st;
  MXQ_REQUIRE(p != nullptr, MXQ_EINVAL, "attn_select_blocks: params is NULL");
  MXQ_REQUIRE(q != nullptr && k != nullptr && mask != nullptr, MXQ_EINVAL,
              "attn_select_blocks: q, k and mask are required");
  MXQ_REQUIRE(p->topk >= 0 || (p->ratio_num >= 0 && p->ratio_den > 0), MXQ_EINVAL,
              "attn_select_blocks: need topk >= 0 or ratio_num >= 0 and ratio_den > 0");
  MXQ_REQUIRE(p->group_shared == 0 || p->group_shared == 1, MXQ_EINVAL,
              "attn_select_blocks: group_shared must be 0 or 1");
  MXQ_REQUIRE(p->heuristic == 0 || p->heuristic == 1, MXQ_EINVAL,
              "attn_select_blocks: heuristic must be 0 (tile means) or 1 (max-pooled key logits)");
  MXQ_REQUIRE(p->sink_tiles >= 0 && p->local_tiles >= 0, MXQ_EINVAL,
              "attn_select_blocks: sink_tiles and local_tiles must be >= 0");
  MXQ_REQUIRE(workspace != nullptr && ws_bytes >= attn_select_blocks_workspace(s), MXQ_EINVAL,
              "attn_select_blocks: workspace too small");
  hipStream_t strm = as_stream(stream);
  const int n_qt = s->N / s->Bq, n_kt = s->N / s->Bk;
  float* qmean = static_cast<float*>(workspace);
  float* kmean = qmean + static_cast<size_t>(s->B) * s->Hq * n_qt * s->D;
  // a zero budget chooses only the forced tiles: without a score request the
  // scores (and the tile means behind them) are not needed
  const bool score_free = scores == nullptr && (p->topk == 0 || (p->topk < 0 && p->ratio_num == 0));
  if (!score_free) {
    hipLaunchKernelGGL(k_tile_means, dim3(n_qt, s->B * s->Hq), dim3(s->D), 0, strm, q, qmean, s->N,
                       s->D, s->Bq, s->n_valid, n_qt, 0);
    if ((st = check_launch("k_tile_means(q)")) != MXQ_OK) return st;
    hipLaunchKernelGGL(k_tile_means, dim3(n_kt, s->B * s->Hkv), dim3(s->D), 0, strm, k, kmean, s->N,
                       s->D, s->Bk, s->n_valid, n_kt, 1);
    if ((st = check_launch("k_tile_means(k)")) != MXQ_OK) return st;
  }
  return launch_select(qmean, kmean, k, s, p, mask, n_fp16, scores, score_free, strm);
}

extern "C" size_t attn_select_lines_workspace(const mxq_attn_shape* s) {
  if (s == nullptr || s->Bq <= 0) return 0;
  const size_t n_qt = static_cast<size_t>(s->N / s->Bq);
  return (static_cast<size_t>(s->B) * s->Hq * n_qt * static_cast<size_t>(s->D) +
          static_cast<size_t>(s->B) * s->Hq * static_cast<size_t>(s->N)) * sizeof(float);
}

extern "C" mxq_status attn_select_lines(const uint16_t* q, const uint16_t* k, const mxq_attn_shape* s,
                                        const mxq_line_params* p, void* workspace, size_t ws_bytes,
                                        int32_t* lines, float* scores, mxq_stream_t stream) {
  mxq_status st = validate_shape(s);
  if (st != MXQ_OK) return st;
  MXQ_REQUIRE(p != nullptr, MXQ_EINVAL, "attn_select_lines: params is NULL");
  MXQ_REQUIRE(p->n_lines >= 0 && p->n_lines <= kMaxLines, MXQ_EINVAL,
              "attn_select_lines: n_lines must be in [0, 16]");
  MXQ_REQUIRE(p->sink_tokens >= 0, MXQ_EINVAL, "attn_select_lines: sink_tokens must be >= 0");
  MXQ_REQUIRE(p->group_shared == 0 || p->group_shared == 1, MXQ_EINVAL,
              "attn_select_lines: group_shared must be 0 or 1");
  if (p->n_lines == 0) return MXQ_OK;
  MXQ_REQUIRE(q != nullptr && k != nullptr && lines != nullptr, MXQ_EINVAL,
              "attn_select_lines: q, k and lines are required");
  MXQ_REQUIRE(workspace != nullptr && ws_bytes >= attn_select_lines_workspace(s), MXQ_EINVAL,
              "attn_select_lines: workspace too small");
  hipStream_t strm = as_stream(stream);
  // every line is a sink token when the list has no room for a scored key (or
  // no key is left to score): without a score request, write it directly
  const int n_first = std::min(std::min(p->sink_tokens, s->n_valid), p->n_lines);
  if (scores == nullptr && (n_first == p->n_lines || n_first == s->n_valid)) {
    const int total = s->B * s->Hq * p->n_lines;
    hipLaunchKernelGGL(k_lines_first, dim3((total + 255) / 256), dim3(256), 0, strm, lines, total, p->n_lines,
                       n_first);
    return check_launch("k_lines_first");
  }
  const int n_qt = s->N / s->Bq;
  float* qmean = static_cast<float*>(workspace);
  hipLaunchKernelGGL(k_tile_means, dim3(n_qt, s->B * s->Hq), dim3(s->D), 0, strm, q, qmean, s->N,
                     s->D, s->Bq, s->n_valid, n_qt, 0);
  if ((st = check_launch("k_tile_means(q)")) != MXQ_OK) return st;
  LineArgs a;
  a.qmean = qmean; a.k = k;
  a.ws_scores = qmean + static_cast<size_t>(s->B) * s->Hq * n_qt * s->D;
  a.scores = scores; a.lines = lines;
  a.Hq = s->Hq; a.Hkv = s->Hkv; a.N = s->N; a.n_valid = s->n_valid; a.D = s->D; a.n_qt = n_qt;
  a.n_vt = (s->n_valid + s->Bq - 1) / s->Bq;
  a.shared = p->group_shared; a.n_lines = p->n_lines; a.sink = p->sink_tokens;
  const int Hsel = a.shared ? s->Hkv : s->Hq;
  hipLaunchKernelGGL(k_line_scores, dim3((s->N + 255) / 256, Hsel, s->B), dim3(256), 0, strm, a);
  if ((st = check_launch("k_line_scores")) != MXQ_OK) return st;
  hipLaunchKernelGGL(k_line_topk, dim3(Hsel, s->B), dim3(256), 0, strm, a);
  return check_launch("k_line_topk");
}

// mxq_quantize: MXFP4 / MXFP8 / INT4-G32 / fp16 conversion of bf16 tensors.
//
// Block-scaled quantisation (ThriftAttention abstract; OCP MX rules for the
// shared E8M0 exponent).  All four conversions are memory-bound: one pass that
// reads each bf16 once and writes the codes once.  Rounding is done with
// compares and integer bit operations so that every code is the exact
// round-half-even of the exactly scaled input.
#include <algorithm>

#include "mxq_internal.h"

// Every product and sum in this file is rounded on its own, as written: with
// contraction off the compiler may not fuse a*b+c into one FMA.  (HIP's
// __fmul_rn/__fadd_rn are plain * and + defined in a header, so they would
// still be fused; plain operators under this pragma are not.)
#pragma clang fp contract(off)

namespace mxq {
namespace {

// One quarter of a 32-element block per lane: the lane's 8 bf16 (element 2i
// in the low half of word i), the four lanes of an aligned quad holding the
// block's quarters in order.  The block maximum is shared across the quad
// with two DPP quad permutes (every lane of the quad must be active); returns
// the lane's 8 E2M1 codes (element 0 in the low nibble) and sets e to the
// block's shared exponent (OCP MX: floor(log2 amax) - 2).  Each element is
// scaled exactly by 2^-e and rounded to the nearest E2M1 magnitude, ties to
// the even code; the sign bit copies the input's.
__device__ __forceinline__ uint32_t mxfp4_quarter(const uint4 w4, int& e) {
  const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    amax = fmaxf(amax, fabsf(__uint_as_float(w[i] << 16)));
    amax = fmaxf(amax, fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
  }
  const int ai = __float_as_int(amax);
  const float a1 = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(ai, 0xB1, 0xF, 0xF, false)));  // quad [1,0,3,2]
  const int a1i = __float_as_int(a1);
  amax = fmaxf(a1, __int_as_float(__builtin_amdgcn_mov_dpp(a1i, 0x4E, 0xF, 0xF, false)));  // quad [2,3,0,1]
  e = shared_exponent(amax, 2);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __builtin_ldexpf(__uint_as_float(w[i] << 16), -e);
    v[2 * i + 1] = __builtin_ldexpf(__uint_as_float(w[i] & 0xFFFF0000u), -e);
  }
  return e2m1_pack8(v);
}

// ---- MXFP4 along D: four lanes per 32-element block ---------------------------
// x [rows][D] bf16 -> codes [rows][D/2], scales [rows][D/32].  Lane 4 blk + u
// takes elements 8u .. 8u+7 of block blk, so each load of a wave reads 1 KB of
// contiguous input and each code store writes 256 contiguous bytes.
// A second tensor (x2, codes2, scales2; n_blocks2 blocks of the same row
// length, N and n_valid) may follow the first in the same launch: blocks
// n_blocks .. n_blocks + n_blocks2 - 1 are its blocks 0 .. n_blocks2 - 1.
__global__ void __launch_bounds__(256) k_quant_mxfp4_d(const uint16_t* __restrict__ x,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       int64_t n_blocks, int64_t blocks_per_row,
                                                       int64_t N, int64_t n_valid,
                                                       const uint16_t* __restrict__ x2 = nullptr,
                                                       uint8_t* __restrict__ codes2 = nullptr,
                                                       uint8_t* __restrict__ scales2 = nullptr,
                                                       int64_t n_blocks2 = 0) {
  // 32-bit indices: the host allows at most 2^29 blocks in one launch
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  uint32_t blk = gid >> 2;
  const int u = static_cast<int>(gid & 3u);
  // no early exit: the quad permutes need every lane of the quad (a quad is
  // one block, so its lanes agree on every condition below)
  const bool in = blk < static_cast<uint32_t>(n_blocks + n_blocks2);
  if (blk >= static_cast<uint32_t>(n_blocks)) {
    blk -= static_cast<uint32_t>(n_blocks);
    x = x2;
    codes = codes2;
    scales = scales2;
  }
  // padding rows (row % N >= n_valid) read as zeros; without padding no
  // division is needed, and power-of-two row lengths and N take shifts
  bool live = in;
  if (n_valid < N) {
    const uint32_t bpr = static_cast<uint32_t>(blocks_per_row), n = static_cast<uint32_t>(N);
    const uint32_t row = (bpr & (bpr - 1)) == 0 ? blk >> __builtin_ctz(bpr) : blk / bpr;
    const uint32_t r = (n & (n - 1)) == 0 ? row & (n - 1) : row % n;
    live = live && r < static_cast<uint32_t>(n_valid);
  }
  const uint4 w4 = live ? reinterpret_cast<const uint4*>(x)[blk * 4u + u] : make_uint4(0, 0, 0, 0);
  int e;
  const uint32_t packed = mxfp4_quarter(w4, e);
  if (in) {
    reinterpret_cast<uint32_t*>(codes)[blk * 4u + u] = packed;
    if (u == 0) scales[blk] = static_cast<uint8_t>(e + 127);
  }
}

// ---- MXFP4 of Q and K plus their tile means in one pass ----------------------
// One workgroup per (head, tile of T rows) of Q (grid x in [0, rows_q)) or K
// (the rest): every 32-element block is quantised as in k_quant_mxfp4_d
// and the bf16 tile is kept in LDS; then thread d sums column d over the
// tile's valid rows in ascending order and divides once by their count, the
// tile mean selection uses (the same operations as its own tile-mean pass, so
// the same bits).  Q means are written [bh][tile][d], K means [bh][d][tile].
template <int D>
__global__ void __launch_bounds__(256) k_quant_mxfp4_tiles(const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales, float* __restrict__ mean,
                                                           int T, int n_tiles, int transposed, int rows_q,
                                                           const uint16_t* __restrict__ x2, uint8_t* __restrict__ codes2,
                                                           uint8_t* __restrict__ scales2, float* __restrict__ mean2,
                                                           int T2, int n_tiles2, int transposed2, int N, int n_valid) {
  __shared__ __attribute__((aligned(16))) uint32_t tile_w[128 * D / 2];  // bf16 pairs, [row][D/2]
  constexpr int BPR = D / 32;  // blocks per row
  int64_t bh = blockIdx.x;
  if (bh >= rows_q) {
    bh -= rows_q;
    x = x2;
    codes = codes2;
    scales = scales2;
    mean = mean2;
    T = T2;
    n_tiles = n_tiles2;
    transposed = transposed2;
  }
  const int tile = blockIdx.y;
  if (tile >= n_tiles) return;  // the whole workgroup
  const int tid = threadIdx.x;
  const int64_t row0 = bh * N + static_cast<int64_t>(tile) * T;  // first row of the tile
  // 16-byte unit tid + 256 p of the tile (row-major, 8 bf16 each), four units
  // to a 32-element block: every load of the tile goes out before any is used
  constexpr int UPR = D / 8;                // units per row
  constexpr int PASSES = 128 * UPR / 256;   // for the tallest tile (128 rows)
  uint4 w4[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int uidx = tid + 256 * p, r = uidx / UPR;
    const bool live = r < T && tile * T + r < n_valid;
    w4[p] = live ? reinterpret_cast<const uint4*>(x + row0 * D)[uidx] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int uidx = tid + 256 * p, r = uidx / UPR;
    if (r < T) *reinterpret_cast<uint4*>(&tile_w[4 * uidx]) = w4[p];
    int e;
    const uint32_t packed = mxfp4_quarter(w4[p], e);  // whole quads agree on r < T
    if (r < T) {
      const int64_t blk = (row0 + r) * BPR + (uidx % UPR) / 4;
      reinterpret_cast<uint32_t*>(codes)[(row0 * D) / 8 + uidx] = packed;
      if ((uidx & 3) == 0) scales[blk] = static_cast<uint8_t>(e + 127);
    }
  }
  __syncthreads();
  if (tid < D) {
    const int rows = max(0, min(T, n_valid - tile * T));
    const uint16_t* col = reinterpret_cast<const uint16_t*>(tile_w) + tid;
    float acc = 0.0f;
    int r = 0;
    for (; r + 16 <= rows; r += 16) {  // 16 LDS reads in flight, then the sums in row order
      uint16_t v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = col[(r + j) * D];
#pragma unroll
      for (int j = 0; j < 16; ++j) acc = acc + bf16_to_f32(v[j]);
    }
    for (; r < rows; ++r) acc = acc + bf16_to_f32(col[r * D]);
    const float m = rows > 0 ? acc / static_cast<float>(rows) : 0.0f;  // correctly rounded division
    if (transposed) mean[(bh * D + tid) * n_tiles + tile] = m;
    else mean[(bh * n_tiles + tile) * D + tid] = m;
  }
}

// ---- MXFP4 of Walsh-Hadamard-rotated rows (reading R34) ---------------------
// x [rows][D] bf16 -> MXFP4 codes and scales of each row times H/sqrt(D).
// D/8 consecutive lanes hold a row, 8 contiguous elements each (one 16-byte
// load per lane).  Butterfly stages h = 1, 2, 4 run inside a lane; stages
// h = 8 ... D/2 pair lane u with lane u ^ (h/8): the lane holding the lower
// index keeps a + b, the other a - b, every sum rounded to fp32 (the same
// values the in-place transform produces, whatever the order of the pairs).
// Then one multiply by fl32(1/sqrt(D)), and each 32-element block (4 lanes)
// is quantised as in k_quant_mxfp4_d.
template <int D>
__global__ void __launch_bounds__(256) k_quant_mxfp4_had(const uint16_t* __restrict__ x,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales, int64_t rows,
                                                         int64_t N, int64_t n_valid,
                                                         const uint16_t* __restrict__ x2,
                                                         uint8_t* __restrict__ codes2,
                                                         uint8_t* __restrict__ scales2, int64_t rows2) {
  constexpr int LPR = D / 8;  // lanes per row
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "power-of-two head_dim");
  // fl32(1/sqrt(D)), the double quotient rounded once to fp32
  constexpr float kInv = D == 32 ? 0x1.6a09e6p-3f : D == 64 ? 0.125f : D == 128 ? 0x1.6a09e6p-4f : 0.0625f;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t row = gid / LPR;
  const int u = static_cast<int>(gid % LPR);
  if (row >= rows) {  // a second tensor may follow in the same launch (whole rows, so whole groups of lanes)
    row -= rows;
    rows = rows2;
    x = x2;
    codes = codes2;
    scales = scales2;
  }
  const bool in = row < rows;
  const bool live = in && (row % N) < n_valid;
  const uint4 w4 = live ? *reinterpret_cast<const uint4*>(x + row * D + 8 * u) : make_uint4(0, 0, 0, 0);
  const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!(i & h)) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __shfl_xor(v[i], m);
      v[i] = (u & m) ? (p - v[i]) : (v[i] + p);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = v[i] * kInv;
    amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int e = shared_exponent(amax, 2);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float s = __builtin_ldexpf(v[i], -e);
    const uint32_t c = e2m1_mag_code(fabsf(s)) | ((__float_as_uint(v[i]) >> 28) & 8u);
    packed |= c << (4 * i);
  }
  if (in) {
    reinterpret_cast<uint32_t*>(codes)[row * (D / 8) + u] = packed;
    if ((u & 3) == 0) scales[row * (D / 32) + u / 4] = static_cast<uint8_t>(e + 127);
  }
}

template <int D>
mxq_status launch_had(const uint16_t* x, uint8_t* codes, uint8_t* scales, int64_t rows, int64_t N,
                      int64_t n_valid, hipStream_t st, const uint16_t* x2 = nullptr, uint8_t* codes2 = nullptr,
                      uint8_t* scales2 = nullptr, int64_t rows2 = 0) {
  const int64_t lanes = (rows + rows2) * (D / 8);
  hipLaunchKernelGGL((k_quant_mxfp4_had<D>), dim3(static_cast<unsigned>((lanes + 255) / 256)), dim3(256), 0, st,
                     x, codes, scales, rows, N, n_valid, x2, codes2, scales2, rows2);
  return check_launch("k_quant_mxfp4_had");
}

// ---- MXFP8 along N (V): x [BH][N][D] -> codes [BH][D][N], scales [BH][D][N/32]
// One thread per (bh, 32-row block, d).  Lanes run over d, so each of the 32
// column loads is a contiguous 128-byte read across the wave.
__global__ void __launch_bounds__(256) k_quant_mxfp8_n(const uint16_t* __restrict__ x,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, int64_t BH,
                                                       int64_t N, int64_t D, int64_t n_valid) {
  int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t nb = N / 32;
  int64_t total = BH * nb * D;
  if (t >= total) return;
  int64_t d = t % D;
  int64_t rest = t / D;
  int64_t blk = rest % nb;
  int64_t bh = rest / nb;
  const uint16_t* col = x + (bh * N + blk * 32) * D + d;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    bool live = blk * 32 + r < n_valid;
    v[r] = live ? bf16_to_f32(col[static_cast<int64_t>(r) * D]) : 0.0f;
    amax = fmaxf(amax, fabsf(v[r]));
  }
  int e = shared_exponent(amax, 8);
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    out[i] = e4m3_pack4(__builtin_ldexpf(v[4 * i], -e), __builtin_ldexpf(v[4 * i + 1], -e),
                        __builtin_ldexpf(v[4 * i + 2], -e), __builtin_ldexpf(v[4 * i + 3], -e));
  uint4* dst = reinterpret_cast<uint4*>(codes + (bh * D + d) * N + blk * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  scales[(bh * D + d) * nb + blk] = static_cast<uint8_t>(e + 127);
}

// ---- fp16, same layout: one thread per 8 elements -----------------------------
__global__ void __launch_bounds__(256) k_to_f16_d(const uint16_t* __restrict__ x,
                                                  uint16_t* __restrict__ y, int64_t n8, int64_t D,
                                                  int64_t N, int64_t n_valid) {
  int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= n8) return;
  int64_t row = (t * 8) / D;
  bool live = (row % N) < n_valid;
  uint4 v = live ? reinterpret_cast<const uint4*>(x)[t] : make_uint4(0, 0, 0, 0);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    _Float16 lo = static_cast<_Float16>(__uint_as_float(w[i] << 16));
    _Float16 hi = static_cast<_Float16>(__uint_as_float(w[i] & 0xFFFF0000u));
    o[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
  }
  reinterpret_cast<uint4*>(y)[t] = make_uint4(o[0], o[1], o[2], o[3]);
}

// ---- fp16 transposed: x [BH][N][D] -> y [BH][D][N], 32x32 tiles via LDS --------
__global__ void __launch_bounds__(256) k_to_f16_n(const uint16_t* __restrict__ x,
                                                  uint16_t* __restrict__ y, int64_t N, int64_t D,
                                                  int64_t n_valid) {
  __shared__ uint16_t tile[32][33];
  int64_t bh = blockIdx.z;
  int64_t n0 = static_cast<int64_t>(blockIdx.x) * 32;
  int64_t d0 = static_cast<int64_t>(blockIdx.y) * 32;
  int tx = threadIdx.x % 32, ty = threadIdx.x / 32;  // 8 rows of 32 per pass
  for (int r = ty; r < 32; r += 8) {
    int64_t n = n0 + r;
    float f = n < n_valid ? bf16_to_f32(x[(bh * N + n) * D + d0 + tx]) : 0.0f;
    tile[r][tx] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) y[(bh * D + d0 + r) * N + n0 + tx] = tile[tx][r];
}

// ---- V^T conversions through an LDS transpose (D <= 256) ---------------------
// x [BH][N][D] bf16 -> fp16 V^T [BH][D][N], or MXFP8 codes [BH][D][N] with
// scales [BH][D][N/32] (blocks of 32 keys).  One workgroup per (bh, KB keys):
// the block's KB rows of D elements are contiguous in x, so they are read in
// one coalesced sweep of 16-byte units; each unit's 8 elements are scattered
// into 8 rows of the transposed tile tt[d][key] (row stride KB + 8 halves,
// 16-byte aligned), and the writers read contiguous keys of one row and store
// 16 bytes at a time.  The arithmetic is that of the per-element kernels
// above, so codes, scales and fp16 values are identical.
// OUT: kVtF16 writes the fp16 copy (to f16), kVtF8 the MXFP8 codes and
// scales, kVtBoth both from the one LDS tile.
constexpr int kVtF16 = 1, kVtF8 = 2, kVtBoth = 3;
template <int KB, int OUT>
__global__ void __launch_bounds__(256) k_vt_n(const uint16_t* __restrict__ x, uint16_t* __restrict__ f16,
                                              uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                              int64_t N, int D, int64_t n_valid, int64_t n_kb) {
  constexpr int S = KB + 8;
  extern __shared__ __attribute__((aligned(16))) uint16_t tt[];  // [D][S]
  const int64_t bh = blockIdx.x / n_kb;
  const int64_t n0 = (blockIdx.x % n_kb) * KB;
  const uint4* src = reinterpret_cast<const uint4*>(x + (bh * N + n0) * D);
  const int cpr = D / 8;  // 16-byte units per key row
  for (int u = threadIdx.x; u < KB * cpr; u += 256) {
    const int key = u / cpr, c = u % cpr;
    const uint4 v = n0 + key < n_valid ? src[u] : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tt[(8 * c + 2 * i) * S + key] = static_cast<uint16_t>(w[i] & 0xFFFFu);
      tt[(8 * c + 2 * i + 1) * S + key] = static_cast<uint16_t>(w[i] >> 16);
    }
  }
  __syncthreads();
  if constexpr ((OUT & kVtF16) != 0) {
    uint16_t* y = f16;
    for (int t = threadIdx.x; t < D * (KB / 8); t += 256) {
      const int d = t / (KB / 8), c = t % (KB / 8);
      const uint4 v = *reinterpret_cast<const uint4*>(tt + d * S + 8 * c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 lo = static_cast<_Float16>(__uint_as_float(w[i] << 16));
        const _Float16 hi = static_cast<_Float16>(__uint_as_float(w[i] & 0xFFFF0000u));
        o[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
      }
      *reinterpret_cast<uint4*>(y + (bh * D + d) * N + n0 + 8 * c) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  if constexpr ((OUT & kVtF8) != 0) {
    for (int t = threadIdx.x; t < D * (KB / 32); t += 256) {
      const int d = t / (KB / 32), b = t % (KB / 32);
      const uint4* r = reinterpret_cast<const uint4*>(tt + d * S + 32 * b);
      float v[32];
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 q = r[i];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
          v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int r2 = 0; r2 < 32; ++r2) amax = fmaxf(amax, fabsf(v[r2]));
      const int e = shared_exponent(amax, 8);
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        o[i] = e4m3_pack4(__builtin_ldexpf(v[4 * i], -e), __builtin_ldexpf(v[4 * i + 1], -e),
                          __builtin_ldexpf(v[4 * i + 2], -e), __builtin_ldexpf(v[4 * i + 3], -e));
      uint4* dst = reinterpret_cast<uint4*>(codes + (bh * D + d) * N + n0 + 32 * b);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
      scales[(bh * D + d) * (N / 32) + n0 / 32 + b] = static_cast<uint8_t>(e + 127);
    }
  }
}

template <int KB, int OUT>
mxq_status launch_vt_n(const uint16_t* x, uint16_t* f16, uint8_t* codes, uint8_t* scales, int64_t BH, int64_t N,
                       int64_t D, int64_t n_valid, hipStream_t st) {
  const int64_t n_kb = N / KB;
  const size_t lds = static_cast<size_t>(D) * (KB + 8) * sizeof(uint16_t);
  hipLaunchKernelGGL((k_vt_n<KB, OUT>), dim3(static_cast<unsigned>(BH * n_kb)), dim3(256), lds, st, x, f16, codes,
                     scales, N, static_cast<int>(D), n_valid, n_kb);
  return check_launch("k_vt_n");
}

// ---- INT4 asymmetric, groups of 32 along D: one thread per group ----------------
__global__ void __launch_bounds__(256) k_quant_int4_d(const uint16_t* __restrict__ x,
                                                      uint8_t* __restrict__ codes,
                                                      uint16_t* __restrict__ scales,
                                                      uint16_t* __restrict__ zeros,
                                                      int64_t n_groups, int64_t groups_per_row,
                                                      int64_t N, int64_t n_valid) {
  int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= n_groups) return;
  int64_t row = g / groups_per_row;
  bool live = (row % N) < n_valid;
  const uint4* src = reinterpret_cast<const uint4*>(x + g * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 q = live ? src[i] : make_uint4(0, 0, 0, 0);
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
  uint32_t packed[4];
  uint16_t sb, zb;
  int4_group(v, packed, sb, zb);
  reinterpret_cast<uint4*>(codes)[g] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  scales[g] = sb;
  zeros[g] = zb;
}

inline unsigned grid_for(int64_t n, int threads) {
  return static_cast<unsigned>(ceil_div(n, threads));
}

}  // namespace
}  // namespace mxq

using namespace mxq;

extern "C" mxq_status mxq_quantize(const uint16_t* x, int64_t B, int64_t H, int64_t N, int64_t D,
                                   int64_t n_valid, mxq_format fmt, mxq_axis axis, void* codes,
                                   void* scales, uint16_t* zeros, mxq_stream_t stream) {
  MXQ_REQUIRE(x != nullptr && codes != nullptr, MXQ_EINVAL, "mxq_quantize: null input or codes");
  MXQ_REQUIRE(B >= 0 && H >= 0 && N >= 0 && D > 0, MXQ_EINVAL, "mxq_quantize: negative shape");
  MXQ_REQUIRE(n_valid >= 0 && n_valid <= N, MXQ_EINVAL, "mxq_quantize: n_valid must be in [0, N]");
  MXQ_REQUIRE(D % 32 == 0, MXQ_EUNSUPPORTED, "mxq_quantize: D must be a multiple of 32");
  MXQ_REQUIRE(axis == MXQ_AXIS_D || axis == MXQ_AXIS_N, MXQ_EINVAL, "mxq_quantize: bad axis");
  MXQ_REQUIRE(axis == MXQ_AXIS_D || N % 32 == 0, MXQ_EUNSUPPORTED,
              "mxq_quantize: AXIS_N needs N to be a multiple of 32");
  hipStream_t st = as_stream(stream);
  const int64_t BH = B * H;
  const int64_t rows = BH * N;
  if (rows == 0) return MXQ_OK;
  if (fmt == MXQ_MXFP4_E2M1 && axis == MXQ_AXIS_D) {
    MXQ_REQUIRE(scales != nullptr && zeros == nullptr, MXQ_EINVAL,
                "mxq_quantize MXFP4: scales required, zeros must be NULL");
    int64_t nb = rows * (D / 32);
    MXQ_REQUIRE(nb <= (int64_t{1} << 29), MXQ_EUNSUPPORTED, "mxq_quantize MXFP4: at most 2^29 blocks of 32");
    hipLaunchKernelGGL(k_quant_mxfp4_d, dim3(grid_for(4 * nb, 256)), dim3(256), 0, st, x,
                       static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales), nb, D / 32, N,
                       n_valid);
    return check_launch("k_quant_mxfp4_d");
  }
  if (fmt == MXQ_MXFP4_E2M1_HADAMARD) {
    MXQ_REQUIRE(axis == MXQ_AXIS_D, MXQ_EUNSUPPORTED, "mxq_quantize MXFP4_HADAMARD: AXIS_D only");
    MXQ_REQUIRE(scales != nullptr && zeros == nullptr, MXQ_EINVAL,
                "mxq_quantize MXFP4_HADAMARD: scales required, zeros must be NULL");
    MXQ_REQUIRE(rows * (D / 8) <= (int64_t{1} << 40), MXQ_EUNSUPPORTED, "mxq_quantize: tensor too large");
    uint8_t* c8 = static_cast<uint8_t*>(codes);
    uint8_t* s8 = static_cast<uint8_t*>(scales);
    switch (D) {
      case 32: return launch_had<32>(x, c8, s8, rows, N, n_valid, st);
      case 64: return launch_had<64>(x, c8, s8, rows, N, n_valid, st);
      case 128: return launch_had<128>(x, c8, s8, rows, N, n_valid, st);
      case 256: return launch_had<256>(x, c8, s8, rows, N, n_valid, st);
      default: return fail(MXQ_EUNSUPPORTED, "mxq_quantize MXFP4_HADAMARD: D must be 32, 64, 128 or 256");
    }
  }
  if (fmt == MXQ_MXFP8_E4M3 && axis == MXQ_AXIS_N) {
    MXQ_REQUIRE(scales != nullptr && zeros == nullptr, MXQ_EINVAL,
                "mxq_quantize MXFP8: scales required, zeros must be NULL");
    MXQ_REQUIRE(N % 128 == 0, MXQ_EUNSUPPORTED, "mxq_quantize MXFP8 AXIS_N: N must be a multiple of 128");
    if (D <= 256 && BH * (N / 64) <= 0x7FFFFFFF)
      return launch_vt_n<64, kVtF8>(x, nullptr, static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales), BH, N,
                                    D, n_valid, st);
    int64_t total = BH * (N / 32) * D;
    hipLaunchKernelGGL(k_quant_mxfp8_n, dim3(grid_for(total, 256)), dim3(256), 0, st, x,
                       static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales), BH, N, D, n_valid);
    return check_launch("k_quant_mxfp8_n");
  }
  if (fmt == MXQ_FP16) {
    MXQ_REQUIRE(scales == nullptr && zeros == nullptr, MXQ_EINVAL,
                "mxq_quantize FP16: scales and zeros must be NULL");
    if (axis == MXQ_AXIS_D) {
      int64_t n8 = rows * D / 8;
      hipLaunchKernelGGL(k_to_f16_d, dim3(grid_for(n8, 256)), dim3(256), 0, st, x,
                         static_cast<uint16_t*>(codes), n8, D, N, n_valid);
      return check_launch("k_to_f16_d");
    }
    if (D <= 256 && BH * (N / 32) <= 0x7FFFFFFF) {
      uint16_t* f16 = static_cast<uint16_t*>(codes);
      if (N % 64 == 0) return launch_vt_n<64, kVtF16>(x, f16, nullptr, nullptr, BH, N, D, n_valid, st);
      return launch_vt_n<32, kVtF16>(x, f16, nullptr, nullptr, BH, N, D, n_valid, st);
    }
    MXQ_REQUIRE(BH <= 65535, MXQ_EUNSUPPORTED, "mxq_quantize FP16 AXIS_N: B*H must be <= 65535");
    hipLaunchKernelGGL(k_to_f16_n, dim3(static_cast<unsigned>(N / 32), static_cast<unsigned>(D / 32),
                                        static_cast<unsigned>(BH)),
                       dim3(256), 0, st, x, static_cast<uint16_t*>(codes), N, D, n_valid);
    return check_launch("k_to_f16_n");
  }
  if (fmt == MXQ_INT4_ASYM_G32 && axis == MXQ_AXIS_D) {
    MXQ_REQUIRE(scales != nullptr && zeros != nullptr, MXQ_EINVAL,
                "mxq_quantize INT4: scales and zeros required");
    int64_t ng = rows * (D / 32);
    hipLaunchKernelGGL(k_quant_int4_d, dim3(grid_for(ng, 256)), dim3(256), 0, st, x,
                       static_cast<uint8_t*>(codes), static_cast<uint16_t*>(scales), zeros, ng,
                       D / 32, N, n_valid);
    return check_launch("k_quant_int4_d");
  }
  return fail(MXQ_EUNSUPPORTED, "mxq_quantize: unsupported (format, axis) pair");
}

extern "C" mxq_status mxq_prefill_operands(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                           const mxq_attn_shape* s, int32_t rotate, uint8_t* q_codes,
                                           uint8_t* q_scales, uint8_t* k_codes, uint8_t* k_scales,
                                           uint8_t* v_codes, uint8_t* v_scales, uint16_t* v_f16t,
                                           mxq_stream_t stream) {
  MXQ_REQUIRE(s != nullptr, MXQ_EINVAL, "mxq_prefill_operands: shape is NULL");
  MXQ_REQUIRE(s->B >= 1 && s->Hq >= 1 && s->Hkv >= 1 && s->N >= 1 && s->n_valid >= 1 && s->n_valid <= s->N,
              MXQ_EINVAL, "mxq_prefill_operands: bad shape");
  MXQ_REQUIRE(s->D == 64 || s->D == 128, MXQ_EUNSUPPORTED, "mxq_prefill_operands: D must be 64 or 128");
  MXQ_REQUIRE(s->N % 128 == 0, MXQ_EUNSUPPORTED, "mxq_prefill_operands: N must be a multiple of 128");
  MXQ_REQUIRE(rotate == 0 || rotate == 1, MXQ_EINVAL, "mxq_prefill_operands: rotate must be 0 or 1");
  const bool qk = q_codes || q_scales || k_codes || k_scales;
  const bool v8 = v_codes || v_scales;
  MXQ_REQUIRE(!qk || (q && k && q_codes && q_scales && k_codes && k_scales), MXQ_EINVAL,
              "mxq_prefill_operands: Q/K outputs need q, k and all four arrays");
  MXQ_REQUIRE(!v8 || (v && v_codes && v_scales), MXQ_EINVAL, "mxq_prefill_operands: V MXFP8 needs v, codes and scales");
  MXQ_REQUIRE(!v_f16t || v, MXQ_EINVAL, "mxq_prefill_operands: the fp16 V^T copy needs v");
  hipStream_t st = as_stream(stream);
  const int64_t D = s->D, N = s->N, nv = s->n_valid;
  const int64_t rows_q = static_cast<int64_t>(s->B) * s->Hq * N, rows_k = static_cast<int64_t>(s->B) * s->Hkv * N;
  mxq_status r = MXQ_OK;
  if (qk) {  // Q and K in one launch
    if (rotate) {
      r = D == 128 ? launch_had<128>(q, q_codes, q_scales, rows_q, N, nv, st, k, k_codes, k_scales, rows_k)
                   : launch_had<64>(q, q_codes, q_scales, rows_q, N, nv, st, k, k_codes, k_scales, rows_k);
    } else {
      const int64_t nb_q = rows_q * (D / 32), nb_k = rows_k * (D / 32);
      MXQ_REQUIRE(nb_q + nb_k <= (int64_t{1} << 29), MXQ_EUNSUPPORTED,
                  "mxq_prefill_operands: at most 2^29 blocks of 32 in Q and K together");
      hipLaunchKernelGGL(k_quant_mxfp4_d, dim3(grid_for(4 * (nb_q + nb_k), 256)), dim3(256), 0, st, q, q_codes, q_scales,
                         nb_q, D / 32, N, nv, k, k_codes, k_scales, nb_k);
      r = check_launch("k_quant_mxfp4_d");
    }
    if (r != MXQ_OK) return r;
  }
  const int64_t BH = static_cast<int64_t>(s->B) * s->Hkv;
  if (v8 && v_f16t) return launch_vt_n<64, kVtBoth>(v, v_f16t, v_codes, v_scales, BH, N, D, nv, st);
  if (v8) return launch_vt_n<64, kVtF8>(v, nullptr, v_codes, v_scales, BH, N, D, nv, st);
  if (v_f16t) return launch_vt_n<64, kVtF16>(v, v_f16t, nullptr, nullptr, BH, N, D, nv, st);
  return MXQ_OK;
}

extern "C" mxq_status mxq_prefill_operands_means(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                                 const mxq_attn_shape* s, uint8_t* q_codes, uint8_t* q_scales,
                                                 uint8_t* k_codes, uint8_t* k_scales, uint8_t* v_codes,
                                                 uint8_t* v_scales, uint16_t* v_f16t, float* q_means,
                                                 float* k_means, mxq_stream_t stream) {
  MXQ_REQUIRE(s != nullptr, MXQ_EINVAL, "mxq_prefill_operands_means: shape is NULL");
  MXQ_REQUIRE(s->B >= 1 && s->Hq >= 1 && s->Hkv >= 1 && s->N >= 1 && s->n_valid >= 1 && s->n_valid <= s->N,
              MXQ_EINVAL, "mxq_prefill_operands_means: bad shape");
  MXQ_REQUIRE(s->D == 64 || s->D == 128, MXQ_EUNSUPPORTED, "mxq_prefill_operands_means: D must be 64 or 128");
  MXQ_REQUIRE(s->N % 128 == 0, MXQ_EUNSUPPORTED, "mxq_prefill_operands_means: N must be a multiple of 128");
  MXQ_REQUIRE((s->Bq == 64 || s->Bq == 128) && (s->Bk == 64 || s->Bk == 128), MXQ_EUNSUPPORTED,
              "mxq_prefill_operands_means: Bq and Bk must be 64 or 128");
  MXQ_REQUIRE(q && k && q_codes && q_scales && k_codes && k_scales && q_means && k_means, MXQ_EINVAL,
              "mxq_prefill_operands_means: q, k, the four Q/K arrays and both mean arrays are required");
  const bool v8 = v_codes || v_scales;
  MXQ_REQUIRE(!v8 || (v && v_codes && v_scales), MXQ_EINVAL,
              "mxq_prefill_operands_means: V MXFP8 needs v, codes and scales");
  MXQ_REQUIRE(!v_f16t || v, MXQ_EINVAL, "mxq_prefill_operands_means: the fp16 V^T copy needs v");
  hipStream_t st = as_stream(stream);
  const int64_t D = s->D, N = s->N, nv = s->n_valid;
  const int64_t rows_q = static_cast<int64_t>(s->B) * s->Hq, rows_k = static_cast<int64_t>(s->B) * s->Hkv;
  MXQ_REQUIRE(rows_q + rows_k <= 0x7FFFFFFF, MXQ_EUNSUPPORTED, "mxq_prefill_operands_means: too many heads");
  const int nt_q = static_cast<int>(N / s->Bq), nt_k = static_cast<int>(N / s->Bk);
  const dim3 grid(static_cast<unsigned>(rows_q + rows_k), static_cast<unsigned>(std::max(nt_q, nt_k)));
  if (D == 128)
    hipLaunchKernelGGL(k_quant_mxfp4_tiles<128>, grid, dim3(256), 0, st, q, q_codes, q_scales, q_means, s->Bq, nt_q,
                       0, static_cast<int>(rows_q), k, k_codes, k_scales, k_means, s->Bk, nt_k, 1,
                       static_cast<int>(N), static_cast<int>(nv));
  else
    hipLaunchKernelGGL(k_quant_mxfp4_tiles<64>, grid, dim3(256), 0, st, q, q_codes, q_scales, q_means, s->Bq, nt_q,
                       0, static_cast<int>(rows_q), k, k_codes, k_scales, k_means, s->Bk, nt_k, 1,
                       static_cast<int>(N), static_cast<int>(nv));
  mxq_status r = check_launch("k_quant_mxfp4_tiles");
  if (r != MXQ_OK) return r;
  const int64_t BH = static_cast<int64_t>(s->B) * s->Hkv;
  if (v8 && v_f16t) return launch_vt_n<64, kVtBoth>(v, v_f16t, v_codes, v_scales, BH, N, D, nv, st);
  if (v8) return launch_vt_n<64, kVtF8>(v, nullptr, v_codes, v_scales, BH, N, D, nv, st);
  if (v_f16t) return launch_vt_n<64, kVtF16>(v, v_f16t, nullptr, nullptr, BH, N, D, nv, st);
  return MXQ_OK;
}

/*
 * mxq.h -- block-scaled low-bit attention with selective mixed precision on
 * AMD Instinct MI355X (gfx950).  C ABI of libmxq.so.
 *
 * The method (what each call computes) comes from these pages:
 *  - ThriftAttention: Selective Mixed Precision for Long-Context FP4 Attention
 *    (abstract): stage 1, a cheap heuristic picks a few important query-key
 *    block pairs for FP16; stage 2 computes those blocks in FP16 and the rest
 *    in FP4 and merges both through one online softmax.
 *  - HyQuant: Hybrid-Precision Quantization for LLM Attention (summary and
 *    abstract): vertical-line (sink) tokens and a local window stay in high
 *    precision; decode compresses the KV cache and fuses dequantisation into
 *    attention.
 *  - "Attention Quantization" topic page (overview): block-scaled FP8/FP4 and
 *    integer formats; softmax stays in full precision.
 *  - NOVA-KV abstract (third page): decode reads the whole KV cache every step,
 *    so it is bandwidth-bound.
 * Formats follow the OCP Microscaling v1.0 rules (E2M1 / E4M3 elements with an
 * E8M0 shared exponent per 32 elements).  Points the pages leave open are
 * settled by numbered readings (R1-R24); each call below states the readings
 * it follows.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers to contiguous row-major arrays that
 *    the caller allocates and owns.  The library never keeps them after the
 *    call returns (work is enqueued on `stream` and runs asynchronously).
 *  - bf16 and fp16 values travel as uint16_t bit patterns; E2M1, E4M3 and
 *    E8M0 as uint8_t.  Two E2M1 codes share a byte: element 2k in bits 0-3,
 *    element 2k+1 in bits 4-7.  An E8M0 byte e means 2^(e-127).
 *  - `stream` is a hipStream_t (NULL = the default stream).
 *  - All arguments are validated on the host before anything is enqueued; on
 *    any error nothing is written.  MXQ_EINVAL: bad argument (null pointer,
 *    inconsistent shape, too-small workspace).  MXQ_EUNSUPPORTED: valid but
 *    not implemented (head_dim other than 64/128, tile sizes, format/axis
 *    pairs).  MXQ_EHIP: a HIP launch error; mxq_last_error() has the text.
 *    Faults inside kernels surface at the caller's next synchronisation.
 *  - Results are deterministic: the same inputs give the same bits.
 *  - Calls are reentrant and hold no state between calls, except the one
 *    fixed device array of attn_quantkv_decode_noalloc (see there).
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* mxq_stream_t; /* a hipStream_t */

typedef enum { MXQ_OK = 0, MXQ_EINVAL = 1, MXQ_EUNSUPPORTED = 2, MXQ_EHIP = 3 } mxq_status;

typedef enum {
  MXQ_MXFP4_E2M1 = 1,   /* E2M1 codes + one E8M0 scale per 32 elements      */
  MXQ_MXFP8_E4M3 = 2,   /* E4M3 codes + one E8M0 scale per 32 elements      */
  MXQ_INT4_ASYM_G32 = 3,/* 4-bit codes + fp16 scale and zero per 32 elements */
  MXQ_FP16 = 4,         /* plain fp16 copy                                  */
  MXQ_MXFP4_E2M1_HADAMARD = 5 /* MXFP4 of each row rotated by H/sqrt(D)     */
} mxq_format;

typedef enum {
  MXQ_AXIS_D = 0, /* blocks run along head_dim; output keeps [.., N, D]         */
  MXQ_AXIS_N = 1  /* blocks run along the sequence; output is [.., D, N]        */
} mxq_axis;

typedef enum { MXQ_MIXED = 0, MXQ_ALL_LOWBIT = 1, MXQ_ALL_FP16 = 2, MXQ_GROUP_HEADS = 16 } mxq_mode;
typedef enum { MXQ_OUT_F32 = 0, MXQ_OUT_BF16 = 1 } mxq_out_dtype;

/* Attention problem.  Q is [B][Hq][N][D], K and V are [B][Hkv][N][D].
 * N: padded length (multiple of 128); n_valid <= N: rows >= n_valid are
 * padding (never attended to, output 0).  D in {64, 128}.  Hq % Hkv == 0; query
 * head h uses kv head h / (Hq/Hkv).  Tiles: Bq in {64, 128} query rows by
 * Bk = 64 keys.  causal: key index <= query index (aligned self-attention). */
typedef struct {
  int32_t B, Hq, Hkv, N, n_valid, D, Bq, Bk, causal;
} mxq_attn_shape;

/* Selection parameters (readings R8-R11).  Per query tile i the FP16 set is
 * the forced tiles (key tiles j < sink_tiles, and the local window: key tiles
 * meeting rows [i*Bq - (local_tiles-1)*Bk, last row of tile i]; none when
 * local_tiles == 0) plus the k_i best-scoring other valid tiles, where
 * k_i = topk if topk >= 0, else ceil(ratio_num * |valid tiles of i| / ratio_den)
 * (integer arithmetic), capped at the number of candidates.  Ties in score go
 * to the lower tile index.  group_shared = 1 (reading R35; HyQuant's
 * vertical-line signals shared by the heads of a group, applied to tiles):
 * the G query heads of a kv group score with their shared tile means (the G
 * heads' means summed in fp32 in head order, divided once by G) and so share
 * one mask; 0: per query head.  heuristic (ThriftAttention, abstract: the
 * importance of each query-key interaction; the pages give no formula):
 * 0, reading R8 (mean of the query tile . mean of the key tile); 1, reading
 * R37, max-pooled key logits: the largest, over the key tile's valid keys, of
 * (mean of the query tile) . key, with R8's fp32 order (a tile with no valid
 * key scores -inf); it needs the key rows, so attn_select_blocks_means takes
 * 0 only. */
typedef struct {
  int32_t topk, ratio_num, ratio_den, sink_tiles, local_tiles;
  int32_t group_shared;
  int32_t heuristic;
} mxq_select_params;

/* ---------------------------------------------------------------------------
 * mxq_quantize -- block-scaled quantisation of a bf16 tensor x [B][H][N][D].
 * ThriftAttention abstract (block-scaled quantisation moves attention to 4-bit);
 * readings R2-R6 (MX rules), R19 (INT4).  Rows n >= n_valid are treated as 0.
 * Supported (fmt, axis) pairs and outputs:
 *  MXFP4_E2M1, AXIS_D: codes u8 [B][H][N][D/2], scales u8 [B][H][N][D/32].
 *     e = floor(log2 amax) - 2 (clamped to [-127,127]; amax 0 -> -127),
 *     code = round-half-even of x*2^-e onto {0,.5,1,1.5,2,3,4,6} (saturating),
 *     sign bit copies the sign of x.
 *  MXFP8_E4M3, AXIS_N: codes u8 [B][H][D][N], scales u8 [B][H][D][N/32]
 *     (blocks of 32 consecutive rows n per column d).  e = floor(log2 amax)-8,
 *     code = OCP E4M3 round-half-even of x*2^-e, saturating at 448.
 *  MXFP4_E2M1_HADAMARD, AXIS_D: as MXFP4 above, of each row times the
 *     orthonormal Walsh-Hadamard matrix H/sqrt(D), Sylvester order (reading
 *     R34: the fast transform with stages h = 1, 2, ..., D/2, each pair
 *     (j, j+h) becoming (a+b, a-b) rounded to fp32, then one fp32 multiply by
 *     fl32(1/sqrt(D))).  The rotation the pages name as the alternative to
 *     promotion: applied to Q and K it keeps QK^T and spreads outlier
 *     channels over each block.  D in {32, 64, 128, 256}.
 *  FP16, AXIS_D: codes u16 [B][H][N][D];  FP16, AXIS_N: codes u16 [B][H][D][N].
 *  INT4_ASYM_G32, AXIS_D: codes u8 [B][H][N][D/2]; scales (fp16) and zeros
 *     (fp16) [B][H][N][D/32]:  s = fp16(fl32(max-min)/15), z = fp16(min),
 *     code = clamp(rint(fl32(x-z)/s), 0, 15), 0 when s == 0.
 * `zeros` must be NULL except for INT4.  N must be a multiple of 32 (128 for
 * AXIS_N); D a multiple of 32.  MXFP4 takes at most 2^29 blocks of 32
 * (MXQ_EUNSUPPORTED beyond; in mxq_prefill_operands, Q and K together).
 * ------------------------------------------------------------------------- */
mxq_status mxq_quantize(const uint16_t* x_bf16, int64_t B, int64_t H, int64_t N, int64_t D,
                        int64_t n_valid, mxq_format fmt, mxq_axis axis, void* codes, void* scales,
                        uint16_t* zeros, mxq_stream_t stream);

/* ---------------------------------------------------------------------------
 * mxq_prefill_operands -- every quantised operand attn_mixed_fwd reads, in two
 * launches, with the values the separate mxq_quantize calls give (the
 * block-scaled low-bit operands of the low-precision tiles, ThriftAttention,
 * abstract, and the "Attention Quantization" topic page's MX formats; the
 * fp16 V of the tiles kept in high precision):
 *   q_codes/q_scales, k_codes/k_scales: MXFP4 AXIS_D of Q [B][Hq][N][D] and K
 *     [B][Hkv][N][D] (MXFP4_E2M1_HADAMARD when rotate = 1), one launch;
 *   v_codes/v_scales: MXFP8 AXIS_N of V [B][Hkv][N][D], and v_f16t the fp16
 *     AXIS_N copy, both written from one read of V.
 * Groups may be left out by passing NULL for all of their arrays (Q/K when
 * the attention runs all-FP16; V's MXFP8 likewise; v_f16t when no FP16 tile
 * or line is used).  Shape as for attn_mixed_fwd (rows >= n_valid are zero);
 * D in {64, 128}, N a multiple of 128.
 * ------------------------------------------------------------------------- */
mxq_status mxq_prefill_operands(const uint16_t* q_bf16, const uint16_t* k_bf16, const uint16_t* v_bf16,
                                const mxq_attn_shape* shape, int32_t rotate, uint8_t* q_codes,
                                uint8_t* q_scales, uint8_t* k_codes, uint8_t* k_scales, uint8_t* v_codes,
                                uint8_t* v_scales, uint16_t* v_f16t, mxq_stream_t stream);

/* ---------------------------------------------------------------------------
 * mxq_prefill_operands_means -- mxq_prefill_operands without rotation, plus
 * the tile means attn_select_blocks scores with (ThriftAttention, abstract:
 * stage 1's cheap importance estimate), taken from the same single read of
 * bf16 Q and K.  Q and K are quantised as mxq_prefill_operands does (the same
 * codes and scales); V likewise.  Tile means, fp32: mean of the valid rows of
 * each tile of shape->Bq query rows (Q) or shape->Bk key rows (K), summed in
 * ascending row order and divided once, exactly as attn_select_blocks computes
 * them, so attn_select_blocks_means on them gives attn_select_blocks's result.
 * Layouts: q_means [B*Hq][N/Bq][D], k_means [B*Hkv][D][N/Bk] (key tiles
 * innermost).  Needs D in {64, 128}, N a multiple of 128, Bq and Bk in
 * {64, 128}; q, k, the four Q/K arrays and both mean arrays are required, the
 * V outputs are optional as in mxq_prefill_operands.  Caller-owned device
 * memory; EINVAL / EUNSUPPORTED on bad arguments, nothing launched then.
 * ------------------------------------------------------------------------- */
mxq_status mxq_prefill_operands_means(const uint16_t* q_bf16, const uint16_t* k_bf16, const uint16_t* v_bf16,
                                      const mxq_attn_shape* shape, uint8_t* q_codes, uint8_t* q_scales,
                                      uint8_t* k_codes, uint8_t* k_scales, uint8_t* v_codes, uint8_t* v_scales,
                                      uint16_t* v_f16t, float* q_means, float* k_means, mxq_stream_t stream);

/* ---------------------------------------------------------------------------
 * attn_select_blocks -- stage 1 of ThriftAttention (abstract): choose the
 * query-key tiles that run in FP16.  Importance estimate (reading R8): the
 * score of tile pair (i, j) is mean(Q rows of tile i) . mean(K rows of tile j)
 * over the bf16 inputs, per query head, with a fixed fp32 operation order
 * (sequential sums over rows, one division by the row count, then a sequential
 * sum over d of rounded products, no fused multiply-add), so results are
 * bit-identical to a plain CPU evaluation.
 * Outputs: mask u32 [B][Hq][N/Bq][ceil((N/Bk)/32)] (bit j%32 of word j/32 set
 * when key tile j is FP16 for that query tile); n_fp16 i32 [B][Hq][N/Bq] or
 * NULL; scores f32 [B][Hq][N/Bq][N/Bk] or NULL (every pair, for inspection).
 * A zero budget (topk = 0, or topk < 0 with ratio_num = 0) promotes only the
 * forced tiles; with scores NULL the scores are then not computed at all (the
 * mask and counts are the same).
 * workspace: device memory of at least attn_select_blocks_workspace(shape)
 * bytes, caller-owned, contents undefined after the call.
 * ------------------------------------------------------------------------- */
size_t attn_select_blocks_workspace(const mxq_attn_shape* shape);
mxq_status attn_select_blocks(const uint16_t* q_bf16, const uint16_t* k_bf16,
                              const mxq_attn_shape* shape, const mxq_select_params* params,
                              void* workspace, size_t ws_bytes, uint32_t* mask, int32_t* n_fp16,
                              float* scores, mxq_stream_t stream);

/* ---------------------------------------------------------------------------
 * attn_select_blocks_means -- attn_select_blocks on tile means already
 * computed (mxq_prefill_operands_means, same layouts): the same scores, mask
 * and counts for the same inputs.  q_means, k_means and mask are required;
 * n_fp16 and scores may be NULL.  Same parameter rules as attn_select_blocks.
 * ------------------------------------------------------------------------- */
mxq_status attn_select_blocks_means(const float* q_means, const float* k_means, const mxq_attn_shape* shape,
                                    const mxq_select_params* params, uint32_t* mask, int32_t* n_fp16,
                                    float* scores, mxq_stream_t stream);

/* ---------------------------------------------------------------------------
 * attn_select_lines -- HyQuant (summary and abstract): a few "vertical-line"
 * tokens, single key positions that queries all along the sequence attend
 * to, stay in full precision.  Signal (reading R28): the probe of a query head
 * is the mean of its valid query tiles' means (Bq rows each, as in
 * attn_select_blocks), summed tile by tile in ascending order and divided
 * once; with group_shared the sum runs over the G query heads of the kv group
 * (head, then tile, ascending) and one line set serves the whole group
 * (reading R31).  Score of key j: probe . k_j, fp32, d ascending, rounded
 * product then rounded sum.  Lines of a head: keys 0 .. sink_tokens-1 (the
 * attention sink or CLS token; fewer if n_valid or n_lines is smaller), then
 * the best-scoring remaining valid keys up to n_lines in all, ties to the
 * lower index, listed ascending and padded with -1.  Bit-identical to a plain
 * CPU evaluation of the same formula.
 * Outputs: lines i32 [B][Hq][n_lines] (rows of one kv group identical when
 * shared); scores f32 [B][Hq][N] or NULL (key scores, -inf for j >= n_valid).
 * When no line is chosen by score (n_lines <= sink_tokens, or no valid key
 * past the sink tokens) and scores is NULL, the list is written without
 * computing any score (the same list).
 * n_lines in [0, 16] (0: nothing is written).  workspace: at least
 * attn_select_lines_workspace(shape) bytes, caller-owned, contents undefined
 * after the call.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t n_lines, sink_tokens, group_shared;
} mxq_line_params;

size_t attn_select_lines_workspace(const mxq_attn_shape* shape);
mxq_status attn_select_lines(const uint16_t* q_bf16, const uint16_t* k_bf16,
                             const mxq_attn_shape* shape, const mxq_line_params* params,
                             void* workspace, size_t ws_bytes, int32_t* lines, float* scores,
                             mxq_stream_t stream);

/* ---------------------------------------------------------------------------
 * attn_mixed_fwd -- stage 2 of ThriftAttention (abstract): one fused pass over
 * the key tiles of each query tile, ascending; selected tiles in FP16, the
 * rest low-bit, merged through one online softmax.  Readings R7, R12-R18:
 *  low-bit tile: S = Q_mxfp4 . K_mxfp4 (exactly rounded fp32 whenever the
 *    per-pair spread of block exponents is <= 18), P = E4M3(2^xq) * 2^-8 with
 *    xq = fl32(S*c + 6152 - m) - 6144 (the exponent on a 2^-11 grid),
 *    V from the MXFP8 copy;
 *  FP16 tile: S = Q_bf16 . K_bf16 (fp32 accumulate), P = fp16(2^(S*c - m)),
 *    V from the fp16 copy;
 *  c = fl32(scale * log2 e); m = running max over tiles so far of
 *  ceil(fl32(rowmax(S_tile) * c)); O and l (the sum of the same quantised P)
 *  are rescaled by 2^(m_old - m_new); out = O / l, lse = ln2 * (m + log2 l).
 * Inputs (from mxq_quantize): q_codes/q_scales and k_codes/k_scales MXFP4
 * AXIS_D; v_codes/v_scales MXFP8 AXIS_N; q_bf16, k_bf16 and v_bf16 the
 * original bf16 [..][N][D]; v_f16t fp16 AXIS_N ([..][D][N]).  The bf16/fp16
 * operands may be NULL in MXQ_ALL_LOWBIT mode; the low-bit operands may be
 * NULL in MXQ_ALL_FP16 mode.  v_bf16 is read only when v_f16t is NULL: then
 * the line keys' V values (below) are its values rounded to fp16 (to nearest,
 * ties to even: the fp16 copy's values), and in MXQ_MIXED mode the caller
 * guarantees that the mask promotes no tile (a promoted tile would read zero
 * V); this spares a step that promotes nothing the fp16 copy of V.  mask
 * (from attn_select_blocks) is needed in MXQ_MIXED mode only.
 * softmax_scale <= 0 means 1/sqrt(D).
 * Vertical lines (HyQuant; readings R29, R30): lines i32 [B][Hq][n_lines]
 * (from attn_select_lines), n_lines in [0, 16], in every mode.  An entry takes
 * part when 0 <= key < n_valid and it exceeds every earlier entry of its row
 * (so -1 padding, repeats and out-of-order or out-of-range values are
 * ignored).  Those keys form one FP16 tile (bf16 Q and K, fp16 V, fp16 P)
 * processed first in the reference order, and they are left out of their
 * key tiles; causal masking applies to them as to any key.  They need q_bf16,
 * k_bf16 and v_f16t or v_bf16 in every mode.  lines may be NULL when n_lines
 * is 0.
 * out: [B][Hq][N][D] fp32 or bf16; lse: f32 [B][Hq][N] or NULL (natural log).
 * Rows >= n_valid: out 0, lse -inf.  With N <= 256 (at most two 128-key
 * chunks) B * Hq may not exceed 2^21 and (B * Hq + 8) * Hq may not exceed
 * 2^32 (MXQ_EUNSUPPORTED).
 * mode may carry MXQ_GROUP_HEADS (ORed into one of the three modes): one
 * workgroup serves the G = Hq / Hkv query heads of a kv group, 128 / G rows of
 * each, and the mask row and line list of the group's first head apply to
 * all G heads -- as attn_select_blocks and attn_select_lines with
 * group_shared write them (HyQuant: selection signals shared across the
 * heads of a GQA group; reading R35).  With such masks and lines the result
 * is bit-identical to the default one-head-per-workgroup launch.  Needs
 * G in {2, 4} and N > 256, else MXQ_EUNSUPPORTED.
 * ------------------------------------------------------------------------- */
mxq_status attn_mixed_fwd(const uint8_t* q_codes, const uint8_t* q_scales,
                          const uint8_t* k_codes, const uint8_t* k_scales,
                          const uint8_t* v_codes, const uint8_t* v_scales,
                          const uint16_t* q_bf16, const uint16_t* k_bf16, const uint16_t* v_f16t,
                          const uint16_t* v_bf16, const uint32_t* mask, const int32_t* lines, int32_t n_lines,
                          const mxq_attn_shape* shape, float softmax_scale,
                          mxq_mode mode, void* out, mxq_out_dtype out_dtype, float* lse,
                          mxq_stream_t stream);

/* ---------------------------------------------------------------------------
 * Quantised KV cache for decode (HyQuant summary/abstract; readings R19, R20).
 * Sequence b has seq_len[b] tokens (device array, 1 <= seq_len[b] <=
 * max_seq_len <= L_cap).  Token t of kv head h is read from
 *   - k_sink/v_sink   fp16 [B][Hkv][n_sink][D]      when t < n_sink,
 *   - k_recent/v_recent fp16 [B][Hkv][n_recent][D]  when t >= seq_len[b]-n_recent
 *     (row r holds token seq_len[b]-n_recent+r),
 *   - k_lines/v_lines fp16 [B][Hkv][n_lines][D] row e when t is entry e of
 *     lines i32 [B][Hkv][n_lines] and that entry counts (reading R33: the
 *     token lies in [n_sink, seq_len[b] - n_recent) and exceeds every earlier
 *     entry of the row) -- vertical-line tokens kept in fp16, HyQuant's
 *     hybrid principle in decode; n_lines in [0, 16], arrays NULL when 0,
 *   - otherwise the INT4 arrays: codes u8 [B][Hkv][L_cap][D/2], scale and zero
 *     fp16 [B][Hkv][L_cap][D/32] (mxq_quantize INT4_ASYM_G32 layout), with
 *     x = fl32(code*s + z).
 * ------------------------------------------------------------------------- */
typedef struct {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint16_t* k_scale;
  const uint16_t* k_zero;
  const uint16_t* v_scale;
  const uint16_t* v_zero;
  const uint16_t* k_sink;
  const uint16_t* v_sink;
  const uint16_t* k_recent;
  const uint16_t* v_recent;
  const int32_t* seq_len;
  int32_t L_cap, n_sink, n_recent;
  const int32_t* lines;
  const uint16_t* k_lines;
  const uint16_t* v_lines;
  int32_t n_lines;
} mxq_kv_cache;

/* ---------------------------------------------------------------------------
 * mxq_kv_lines_from_prefill -- the decode cache's vertical-line tokens chosen
 * by importance at prefill (HyQuant, abstract: the prefill's hybrid principle
 * applied to KV-cache compression in decode; reading R36): the lists
 * attn_select_lines wrote with group_shared = 1 (lines_hq i32 [B][Hq][n],
 * identical for the G query heads of a kv group) become the cache's lists
 * lines i32 [B][Hkv][n] (the group's first query head), and the listed
 * tokens' rows of the prompt's K and V (bf16 [B][Hkv][L][D]) are written in
 * fp16 (round to nearest even) to k_lines, v_lines [B][Hkv][n][D]; an entry
 * outside [0, L) gets zero rows (it never takes part, reading R33).  These
 * are the lines, k_lines, v_lines and n_lines of mxq_kv_cache.  n in [1, 16];
 * D a multiple of 8.  Caller-owned device memory; EINVAL on bad arguments,
 * nothing launched then.
 * ------------------------------------------------------------------------- */
mxq_status mxq_kv_lines_from_prefill(const int32_t* lines_hq, int32_t Hq, const uint16_t* k_bf16,
                                     const uint16_t* v_bf16, int32_t B, int32_t Hkv, int32_t L, int32_t D,
                                     int32_t n_lines, int32_t* lines, uint16_t* k_lines, uint16_t* v_lines,
                                     mxq_stream_t stream);

/* ---------------------------------------------------------------------------
 * attn_quantkv_decode -- one decode step: for each sequence b and query head
 * h, softmax(q . k * scale) . v over the cache (fp32 softmax and accumulation,
 * P not quantised), with dequantisation fused into the attention (HyQuant
 * abstract).  The keys of each (b, kv head) are split into num_splits ranges
 * processed independently and merged in ascending split order (reading R23);
 * num_splits 0 picks a value.  q: bf16 [B][Hq][D]; out: f32 [B][Hq][D].
 * workspace: at least attn_quantkv_decode_workspace(...) bytes (caller-owned,
 * contents undefined after the call).  Supported: D = 128; Hq / Hkv in
 * {1, 2, 4}; L_cap <= 2^25.  MXQ_EUNSUPPORTED otherwise.
 * Rounding: scores and the fp32 softmax follow the reference arithmetic up to
 * fp32 accumulation order; the weights p * scale enter the value product in
 * fp16 (relative rounding 2^-11 each), so outputs differ from an all-fp32
 * evaluation by about 1e-4 at unit-variance values.
 * ------------------------------------------------------------------------- */
size_t attn_quantkv_decode_workspace(int32_t B, int32_t Hq, int32_t D, int32_t num_splits,
                                     int32_t max_seq_len);
mxq_status attn_quantkv_decode(const uint16_t* q_bf16, const mxq_kv_cache* cache, int32_t B,
                               int32_t Hq, int32_t Hkv, int32_t D, int32_t max_seq_len,
                               float softmax_scale, int32_t num_splits, void* workspace,
                               size_t ws_bytes, float* out, mxq_stream_t stream);

/* ---------------------------------------------------------------------------
 * attn_quantkv_decode_noalloc -- attn_quantkv_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and the same results, bit
 * for bit, with the split partials held in a fixed array inside the library
 * instead of a caller workspace.  It allocates nothing and calls no allocating
 * routine.
 * Limit: attn_quantkv_decode_workspace(B, Hq, D, num_splits, max_seq_len) must
 * not exceed MXQ_DECODE_SCRATCH_BYTES (16 MiB: e.g. 64 sequences x 32 query
 * heads at the default 8 + 1 splits of a 32768-token cache take 9.6 MB);
 * larger requests return MXQ_EINVAL with nothing launched.
 * Each GPU holds one copy of the array for the life of the process, shared by
 * every call on that GPU: calls that overlap on one GPU (other streams, other
 * host threads) race on it and must be serialised by the caller.  No contents
 * need clearing between calls (every split writes its whole partial).
 * Arguments, layouts and errors otherwise as attn_quantkv_decode.
 * ------------------------------------------------------------------------- */
#define MXQ_DECODE_SCRATCH_BYTES (16u << 20)
mxq_status attn_quantkv_decode_noalloc(const uint16_t* q_bf16, const mxq_kv_cache* cache, int32_t B,
                                       int32_t Hq, int32_t Hkv, int32_t D, int32_t max_seq_len,
                                       float softmax_scale, int32_t num_splits, float* out,
                                       mxq_stream_t stream);

/* ---------------------------------------------------------------------------
 * attn_quantkv_append -- one decode step's cache update (HyQuant summary and
 * abstract: the hybrid principle applied to KV-cache compression; reading
 * R32).  For every sequence b, token t = seq_len[b] (k_new, v_new: bf16
 * [B][Hkv][D], device) enters the fp16 recent window as its last row (the
 * rows move up by one, row r then holds token t+1-n_recent+r), and the row
 * that leaves, token t - n_recent, is quantised to INT4 from its fp16 copy
 * at position t - n_recent unless it is a sink token (t - n_recent < n_sink).
 * With n_recent = 0 the new token itself is quantised (from its fp16
 * rounding) at position t.  A token t < n_sink is also written to the sink
 * copy.  seq_len[b] then becomes t + 1.  The cache layout is the one
 * attn_quantkv_decode reads (mxq_kv_cache, whose vertical-line rows need no
 * update: they hold fixed tokens); the pointers here are writable.
 * A sequence with seq_len[b] outside [0, L_cap) is left unchanged (device
 * data cannot be checked on the host).  D a multiple of 32, at most 256.
 * Calls on one cache must not overlap (they read and write seq_len).
 * ------------------------------------------------------------------------- */
typedef struct {
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint16_t* k_scale;
  uint16_t* k_zero;
  uint16_t* v_scale;
  uint16_t* v_zero;
  uint16_t* k_sink;
  uint16_t* v_sink;
  uint16_t* k_recent;
  uint16_t* v_recent;
  int32_t* seq_len;
  int32_t L_cap, n_sink, n_recent;
} mxq_kv_cache_rw;

mxq_status attn_quantkv_append(const uint16_t* k_new_bf16, const uint16_t* v_new_bf16,
                               const mxq_kv_cache_rw* cache, int32_t B, int32_t Hkv, int32_t D,
                               mxq_stream_t stream);

/* Status text, and the message of the last failing call on this thread. */
const char* mxq_status_string(mxq_status s);
const char* mxq_last_error(void);
/* Library version string. */
const char* mxq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MXQ_H */

/*
 * lamp.h -- C ABI of the mixed-precision tiled attention prefill library
 * (HIP, gfx950 / MI355X).
 *
 * The library computes a FlashAttention-style prefill forward pass in which
 * every QK^T score tile takes one of two paths, both feeding one shared
 * online-softmax state (running maximum m, normaliser l, accumulator O):
 *
 *   8-bit path  Q and K quantised per block (int8 or OCP e4m3) with one fp32
 *               scale per block; 8-bit MFMA; logits rescaled by
 *               sQ * sK * sm_scale; optionally the max-shifted logit and its
 *               exponential rounded to e4m3 ("exp8"); optionally, with exp8,
 *               P V as an fp8 product with e4m3 V tiles ("pv8").
 *   16-bit path Q and K in bf16/fp16; 16-bit MFMA.
 *
 * Sources (pages, by title and section):
 *   - "TileMix: Mixed-Precision Attention for Faster LLM Prefill",
 *     section 2: score tiles (The Tile Architecture), packed per-query-row
 *     bitmask with one bit per group of key tiles, 0 = 16-bit, 1 = 8-bit
 *     (Packed Bitmasks), in-loop dispatch and per-block scale factors
 *     feeding a shared online-softmax state (The Dual-Path Engine);
 *     section 4: grouped-query attention.
 *   - "LampAttention: Look-Ahead Mixed-Precision FlashAttention for Dedicated
 *     Accelerators", Abstract: 8-bit products and exponentials, adaptive
 *     identification of sensitive sub-blocks and their 16-bit recompute.
 *
 * Conventions for every entry point:
 *   - Every data pointer is a DEVICE pointer owned by the caller (the one
 *     exception, lamp_build_mask_per_head's fraction array, says so).  The
 *     library allocates no memory, keeps no state other than a thread-local
 *     error string, never synchronises, and enqueues its kernels on `stream`
 *     (a hipStream_t; NULL = the null stream).
 *   - Arguments are validated synchronously on the host before anything is
 *     launched; on error nothing is enqueued and the call returns a non-zero
 *     lamp_status whose detail is in lamp_last_error().
 *   - Device faults surface at the caller's next synchronisation.
 *   - Sizes are element counts; strides are in elements; the innermost (head
 *     dim) stride is 1.
 *   - A call with an empty problem (any of B, H, S equal to 0) validates its
 *     arguments and returns LAMP_OK without launching.
 */
#ifndef LAMP_H_
#define LAMP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LAMP_ABI_VERSION 3

typedef enum {
  LAMP_OK = 0,
  LAMP_ERR_NULL = 1,        /* a required pointer is NULL                      */
  LAMP_ERR_SHAPE = 2,       /* negative / inconsistent sizes or strides        */
  LAMP_ERR_UNSUPPORTED = 3, /* a valid request this build does not implement   */
  LAMP_ERR_ALIGN = 4,       /* pointer or row stride not 16-byte aligned       */
  LAMP_ERR_HIP = 5          /* the HIP runtime refused a launch                */
} lamp_status;

typedef enum { LAMP_F16 = 0, LAMP_BF16 = 1, LAMP_I8 = 2, LAMP_E4M3 = 3 } lamp_dtype;

typedef enum {
  LAMP_MODE_MASK = 0,       /* TileMix: route by the packed mask only          */
  LAMP_MODE_ADAPTIVE = 1    /* LampAttention: mask, then look-ahead flags      */
} lamp_mode;

/*
 * lamp_quantize_blocks -- per-block absmax quantisation of Q or K.
 *
 * Source: TileMix page, section 2 "The Dual-Path Engine" (queries and keys
 * quantised, products rescaled with per-block scale factors); LampAttention
 * abstract (8-bit floating-point format).
 *
 * x       [B, H, S, D] 16-bit (x_dtype LAMP_F16 or LAMP_BF16) at element
 *         strides (sb, sh, ss, 1); 16-byte aligned, ss a multiple of 8.
 * block   `block_rows` consecutive rows of one (b, h) times all D columns
 *         (use tile_m for Q and tile_n for K); the last block of a sequence
 *         may be short.  1 <= block_rows <= 256.
 * scale   a = max |x| over the block; a == 0 gives scale 0 and all codes 0;
 *         otherwise, in fp32 with round-to-nearest-even,
 *           scale = a / QMAX, inv = QMAX / a, y = x * inv,
 *         QMAX = 127 (LAMP_I8) or 448 (LAMP_E4M3).
 * codes   [B, H, S, D] contiguous, one byte each, 16-byte aligned:
 *           LAMP_I8:   clamp(round_half_even(y), -127, 127) (two's complement)
 *           LAMP_E4M3: OCP E4M3FN bits of y, round-half-even, |y| <= 448.
 * scales  [B, H, ceil(S / block_rows)] fp32 contiguous.
 * D       64, 128 or 256.
 */
lamp_status lamp_quantize_blocks(const void* x, int32_t x_dtype, int64_t B, int64_t H,
                                 int64_t S, int64_t D, int64_t sb, int64_t sh, int64_t ss,
                                 int32_t block_rows, int32_t code_dtype, void* codes,
                                 float* scales, void* stream);

/*
 * lamp_quantize_blocks_varlen -- lamp_quantize_blocks over a variable-length
 * batch.
 *
 * Source: TileMix page, section 4 (variable-length batches), with the
 * quantiser of section 2.  seqlens [B] int32 (device, 4-byte aligned; NULL =
 * every sequence has length S): sequence b occupies rows 0 .. L-1 of its
 * padded [S, D] slice, L = seqlens[b] clamped to [0, S].  Rows L .. S-1 are
 * padding: they are not read, count as zeros for the block absmax, and get
 * code 0 (a block wholly in the padding gets scale 0).  Everything else as
 * for lamp_quantize_blocks.
 */
lamp_status lamp_quantize_blocks_varlen(const void* x, int32_t x_dtype, int64_t B, int64_t H,
                                        int64_t S, int64_t D, int64_t sb, int64_t sh,
                                        int64_t ss, const int32_t* seqlens, int32_t block_rows,
                                        int32_t code_dtype, void* codes, float* scales,
                                        void* stream);

/*
 * lamp_quantize_v_tiles -- V as e4m3 codes for the optional 8-bit P V
 * product (lamp_attn_params.pv8).
 *
 * Source: LampAttention abstract (products evaluated in 8-bit formats).  The
 * pages quantise only Q and K; the 8-bit P V product is a variant whose
 * reading is stated here.  A block is 64 consecutive keys of one (b, h) times
 * all D columns.  With a = max |v| over the block, the scale is 2^e, e the
 * smallest integer with a <= 448 * 2^e, clamped to [-126, 126] (e = 0 for an
 * all-zero block); code = E4M3(v * 2^-e), round-half-even (the scaling is
 * exact, no value saturates).  The power-of-two scale is what the gfx950
 * scaled matrix instruction applies exactly.
 *
 * v        [B, H, S, D] 16-bit (v_dtype LAMP_F16 or LAMP_BF16) at element
 *          strides (sb, sh, ss, 1); 16-byte aligned, strides multiples of 8.
 * seqlens  [B] int32 (device, 4-byte aligned) or NULL: keys at or past
 *          seqlens[b] (clamped to [0, S]) are padding, count as zeros and
 *          get code 0.
 * codes    tile-packed, [B, H, ceil(S / 64), D, 64] bytes, 16-byte aligned:
 *          tile t, row d, position j = 32 c + p (c in {0, 1}, p < 32) holds
 *          the code of key 64 t + 32 (p / 16) + 8 ((p % 16) / 4) + p % 4 + 4 c,
 *          column d (keys past S: 0).  This is the order in which the
 *          kernel's score registers hold a row's 64 keys.
 * scales   [B, H, ceil(S / 64)] fp32, each exactly 2^e.
 * D        64, 128 or 256.
 */
lamp_status lamp_quantize_v_tiles(const void* v, int32_t v_dtype, int64_t B, int64_t H,
                                  int64_t S, int64_t D, int64_t sb, int64_t sh, int64_t ss,
                                  const int32_t* seqlens, void* codes, float* scales,
                                  void* stream);

/*
 * lamp_build_mask -- the random packed precision mask.
 *
 * Source: TileMix page, section 2 "Packed Bitmasks".  One mask row per query
 * tile of tile_m rows; group g covers key tiles [g*G, (g+1)*G) with
 * G = tiles_per_bit, n_g = ceil(ceil(S_k / tile_n) / G) groups; the row is
 * `words_per_row` uint64 words, bit g % 64 of word g / 64 (LSB first), bit 1
 * = 8-bit path, 0 = 16-bit path, unused bits 0.
 *
 * Template: every (b, h, qt, g) is drawn independently.  r = output number
 * ((b*Hq + h)*n_qt + qt)*n_g + g of SplitMix64 (Steele, Lea & Flood 2014)
 * seeded with `seed`; the group is 16-bit iff (r >> 32) < floor(frac_16bit *
 * 2^32).  frac_16bit in [0, 1].
 *
 * mask    [B, Hq, ceil(S_q / tile_m), words_per_row] uint64, 8-byte aligned;
 *         words_per_row >= ceil(n_g / 64).
 */
lamp_status lamp_build_mask(int64_t B, int64_t Hq, int64_t S_q, int64_t S_k, int32_t tile_m,
                            int32_t tile_n, int32_t tiles_per_bit, double frac_16bit,
                            uint64_t seed, uint64_t* mask, int32_t words_per_row,
                            void* stream);

/*
 * lamp_build_mask_per_head -- lamp_build_mask with one 16-bit fraction per
 * query head (per-head mix ratios; a per-layer ratio is one call per layer).
 *
 * Source: TileMix page, section 2 "Packed Bitmasks" (the mask policy is
 * static and chosen per model).  frac_16bit: host array [Hq], each in
 * [0, 1]; query head h uses the threshold floor(frac_16bit[h] * 2^32) with
 * the same SplitMix64 draws as lamp_build_mask.  Hq <= 128.  Everything else
 * as for lamp_build_mask.
 */
lamp_status lamp_build_mask_per_head(int64_t B, int64_t Hq, int64_t S_q, int64_t S_k,
                                     int32_t tile_m, int32_t tile_n, int32_t tiles_per_bit,
                                     const double* frac_16bit, uint64_t seed, uint64_t* mask,
                                     int32_t words_per_row, void* stream);

/*
 * lamp_build_mask_template -- a structured static packed precision mask.
 *
 * Source: TileMix page, section 4 "Why It Matters" (the routing policy is
 * static, data-free structured templates) and section 3 (a "SpTrans75"
 * configuration, named but not defined).  Reading taken: the fixed local and
 * strided patterns of sparse transformers plus attention-sink groups, at
 * group granularity.  Layout, group definition and bit polarity as for
 * lamp_build_mask.  For query tile qt let
 *   pos = (qt + 1) * tile_m - 1 + S_k - S_q
 * (the key position of the tile's last row, queries aligned with the end of
 * the keys as for causal attention), gq = clamp(floor(pos / (tiles_per_bit *
 * tile_n)), 0, n_g - 1) and d = |gq - g|; group g is 16-bit (bit 0) iff
 *   g < sink_groups, or d < band_groups, or (stride_groups > 0 and
 *   d % stride_groups == 0),
 * and 8-bit (bit 1) otherwise; every (b, h) gets the same rows.
 * sink_groups, band_groups, stride_groups >= 0 (LAMP_ERR_SHAPE otherwise).
 *
 * mask    [B, Hq, ceil(S_q / tile_m), words_per_row] uint64, 8-byte aligned;
 *         words_per_row >= ceil(n_g / 64).
 */
lamp_status lamp_build_mask_template(int64_t B, int64_t Hq, int64_t S_q, int64_t S_k,
                                     int32_t tile_m, int32_t tile_n, int32_t tiles_per_bit,
                                     int32_t sink_groups, int32_t band_groups,
                                     int32_t stride_groups, uint64_t* mask,
                                     int32_t words_per_row, void* stream);

/*
 * lamp_attn_fwd -- the dual-path fused attention forward.
 *
 * Sources: TileMix page, section 2 (tile loop, per-group dispatch, shared
 * online softmax) and section 4 (grouped-query attention); LampAttention
 * abstract (8-bit exponentials, adaptive sub-block recompute in 16 bits).
 *
 * For query row i of head h (KV head h / (Hq / Hkv)) and key j:
 *   valid(i, j)  = j < S_k, and j <= i + S_k - S_q when causal (then
 *                  S_q <= S_k: the queries are the last S_q positions, as
 *                  for a chunk of new tokens after S_k - S_q earlier ones);
 *   route8(i, j) = mask bit of (b, h, i / tile_m, (j / tile_n) / G);
 *   s16 = sm * q_i . k_j            s8 = (cq_i . ck_j) * sQ * sK * sm.
 * MODE_MASK, exp8 = 0: O_i = softmax over valid j of the routed logits, times V.
 * Otherwise key tiles are processed in ascending order with the state
 * (m, l, acc) updated after each tile of tile_n = 64 keys:
 *   - ADAPTIVE, 8-bit-routed tile: m' = max(m, rowmax s8); the sub-block of
 *     sub_rows = 32 rows is flagged iff some valid s8_ij - m'_i >= -tau, and
 *     then uses s16 for all its elements in this tile;
 *   - m_new = max(m, rowmax s); alpha = exp(m - m_new);
 *   - p = exp(s - m_new) on 16-bit elements; on 8-bit elements
 *     p = e4m3(exp(e4m3(max(s - m_new, -448)))) when exp8, else exp(s - m_new);
 *   - l = alpha*l + sum p;  acc = alpha*acc + p V;  O = acc / l at the end.
 * P V runs at 16 bits on both paths, unless pv8 = 1 (a variant the pages do
 * not specify; needs exp8 = 1 and MODE_MASK): then on 8-bit tiles the e4m3
 * weights p multiply V codes from lamp_quantize_v_tiles,
 *     acc = alpha*acc + sum_j p_ij * code_j * 2^e(tile),
 * in an fp8 x fp8 matrix product with fp32 accumulation; 16-bit tiles keep
 * the 16-bit V.  v8 [B, Hkv, ceil(S_k/64), D, 64] and v_scale
 * [B, Hkv, ceil(S_k/64)] are then required.
 *
 * Supported: D in {64, 128, 256}; tile_m in {64, 128}; tile_n == 64;
 * in_dtype LAMP_F16 or LAMP_BF16 (q, k, v, out share it); code_dtype LAMP_I8
 * or LAMP_E4M3; sub_rows == 32 in ADAPTIVE mode; Hq % Hkv == 0.
 *
 * Pointers (device): q/k/v/out 16-byte aligned with row strides multiple of
 * 8 elements; q8 [B, Hq, S_q, D] and k8 [B, Hkv, S_k, D] contiguous codes
 * and q_scale [B, Hq, ceil(S_q/tile_m)], k_scale [B, Hkv, ceil(S_k/64)] as
 * written by lamp_quantize_blocks (block_rows tile_m and 64); mask as
 * written by lamp_build_mask.
 * Optional outputs (NULL = not written):
 *   lse        [B, Hq, S_q] fp32, natural-log sum exp of the logits;
 *   flags_out  [B, Hq, ceil(S_q/32), ceil(ceil(S_k/64)/64)] uint64, ADAPTIVE:
 *              bit kt % 64 of word kt / 64 set iff the sub-block was flagged
 *              at key tile kt (all other bits 0);
 *   dbg_qk_acc [B, Hq, S_q, S_k] int32, int8 path only: the raw int32 QK^T
 *              accumulators of every 8-bit key tile a 32-row wave computes
 *              (tiny shapes; other entries are left untouched).
 * Variable-length batch (TileMix section 4; NULL = all lengths S_q / S_k):
 *   seqlens_q, seqlens_k [B] int32 (device, 4-byte aligned): sequence b has
 *   Lq = seqlens_q[b] queries and Lk = seqlens_k[b] keys (clamped to [0, S_q]
 *   and [0, S_k]) at the start of its padded slices; the codes and scales
 *   must come from lamp_quantize_blocks_varlen with the same lengths.
 *   valid(i, j) then reads j < Lk, and j <= i + Lk - Lq when causal (the
 *   caller keeps Lq <= Lk).  A row with no valid key gets O = 0 and LSE =
 *   -inf.  Rows i >= Lq of out, lse and flags_out are not written.
 */
typedef struct {
  uint32_t struct_size;     /* = sizeof(lamp_attn_params); ABI guard         */
  int32_t mode;             /* lamp_mode                                     */
  int32_t causal;           /* 0 / 1                                         */
  float sm_scale;           /* <= 0 selects 1/sqrt(D)                        */
  int64_t B, Hq, Hkv, S_q, S_k, D;
  const void* q;            /* [B, Hq, S_q, D]                               */
  const void* k;            /* [B, Hkv, S_k, D]                              */
  const void* v;            /* [B, Hkv, S_k, D]                              */
  int32_t in_dtype;         /* lamp_dtype: LAMP_F16 | LAMP_BF16              */
  int32_t code_dtype;       /* lamp_dtype: LAMP_I8 | LAMP_E4M3               */
  int64_t q_str[3], k_str[3], v_str[3], o_str[3]; /* (batch, head, row)      */
  const void* q8;
  const void* k8;
  const float* q_scale;
  const float* k_scale;
  const uint64_t* mask;
  int32_t words_per_row;
  int32_t tile_m, tile_n, tiles_per_bit;
  int32_t exp8;             /* 1: 8-bit logit and exp on the 8-bit path      */
  float tau;                /* ADAPTIVE threshold (natural-log units)        */
  int32_t sub_rows;         /* ADAPTIVE sub-block rows (32)                  */
  void* out;                /* [B, Hq, S_q, D] in_dtype                      */
  float* lse;               /* optional                                      */
  uint64_t* flags_out;      /* optional, ADAPTIVE                            */
  int32_t* dbg_qk_acc;      /* optional, int8 path                           */
  const int32_t* seqlens_q; /* optional [B], variable-length batch           */
  const int32_t* seqlens_k; /* optional [B]                                  */
  int32_t pv8;              /* 1: 8-bit P V on 8-bit tiles (exp8, MODE_MASK) */
  const void* v8;           /* pv8: tile-packed V codes                      */
  const float* v_scale;     /* pv8: V block scales (powers of two)           */
} lamp_attn_params;

lamp_status lamp_attn_fwd(const lamp_attn_params* p, void* stream);

/*
 * lamp_decode_fwd -- attention of a few new queries over an int8 key/value
 * cache (decode).
 *
 * Source: TileMix page, section 4 "Why It Matters" (INT8 key/value caches for
 * the decode phase).  Reading taken: the cache holds K and V as int8 codes
 * with one fp32 scale per block of 64 keys of one (b, kv head), as
 * lamp_quantize_blocks writes them (block_rows 64); the queries' codes and
 * scales come from lamp_quantize_blocks (block_rows tile_m).  For query row i
 * of head h (KV head h / (Hq / Hkv)):
 *   s_ij = (cq_i . ck_j) * sQ[i / tile_m] * sK[j / 64] * sm,
 *   O_i  = sum_j softmax_j(s_i) * sV[j / 64] * cv_j,
 * over valid j: j < S_k, and j <= i + S_k - S_q when causal (S_q <= S_k).
 * The GPU rounds p * sV to 16 bits for the P V product.
 *
 * Supported: D in {64, 128}; LAMP_I8 codes; Hq % Hkv == 0 and
 * (Hq / Hkv) * S_q <= 32 (the query group of one KV head fits one 32-column
 * MFMA block); out_dtype LAMP_F16 or LAMP_BF16.
 *
 * Pointers (device): q8 [B, Hq, S_q, D], k8 / v8 [B, Hkv, S_k, D] contiguous
 * 16-byte aligned codes; q_scale [B, Hq, ceil(S_q / tile_m)], k_scale /
 * v_scale [B, Hkv, ceil(S_k / 64)]; out [B, Hq, S_q, D] 16-bit at element
 * strides o_str, head dim contiguous; lse optional [B, Hq, S_q] fp32
 * (natural log).  workspace: caller-owned device
 * memory of at least lamp_decode_workspace_bytes(B, Hkv, S_k, D) bytes,
 * 16-byte aligned (split partials; contents on entry do not matter).
 */
typedef struct {
  uint32_t struct_size;     /* = sizeof(lamp_decode_params); ABI guard       */
  int32_t causal;           /* 0 / 1                                         */
  float sm_scale;           /* <= 0 selects 1/sqrt(D)                        */
  int32_t out_dtype;        /* lamp_dtype: LAMP_F16 | LAMP_BF16              */
  int64_t B, Hq, Hkv, S_q, S_k, D;
  const void* q8;
  const float* q_scale;
  int32_t tile_m;           /* rows per Q scale block                        */
  const void* k8;
  const float* k_scale;
  const void* v8;
  const float* v_scale;
  void* out;
  int64_t o_str[3];         /* (batch, head, row) element strides           */
  float* lse;               /* optional                                      */
} lamp_decode_params;

/* Workspace bytes lamp_decode_fwd needs for these sizes: 0 if a size is
 * negative, SIZE_MAX for sizes no call accepts (S_k above 2^20, D above 256,
 * or B * Hkv above 2^31 - 1). */
size_t lamp_decode_workspace_bytes(int64_t B, int64_t Hkv, int64_t S_k, int64_t D);

lamp_status lamp_decode_fwd(const lamp_decode_params* p, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * lamp_decode_fwd_noalloc -- lamp_decode_fwd without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The split partials go to a fixed scratch array inside the library, one
 * copy per GPU, LAMP_DECODE_SCRATCH_BYTES (32 MiB) in size, held from the
 * first call on that GPU until the process ends (its device address is
 * looked up on that first call).  The call allocates nothing.  Sizes whose
 * partials (lamp_decode_workspace_bytes) exceed the scratch return
 * LAMP_ERR_UNSUPPORTED.  Every call on one GPU shares that GPU's scratch:
 * calls that may overlap on one GPU (different streams, or host threads)
 * race and give undefined results; calls ordered on one stream are safe.
 * The scratch keeps the last call's partials; nothing in it needs to start
 * at zero.  Everything else as for lamp_decode_fwd.
 */
#define LAMP_DECODE_SCRATCH_BYTES (32u << 20)
lamp_status lamp_decode_fwd_noalloc(const lamp_decode_params* p, void* stream);

/*
 * lamp_exp8_table -- the attention kernel's 8-bit exponential of every e4m3
 * code ("LampAttention: Look-Ahead Mixed-Precision FlashAttention for
 * Dedicated Accelerators", Abstract: exponentials evaluated in 8-bit
 * formats).  table: device pointer to 256 bytes; table[c] =
 * E4M3(exp(value(c))) as the kernel computes it (value decoded by the
 * hardware conversion, exp through exp2, rounded to e4m3), except
 * table[0xFF] = 0: 0xFF is the code the fp32 -> e4m3 conversion gives a
 * weight's logit below -464, -inf or NaN, and such a logit weighs 0 as one
 * clamped to -448 would.  With 8-bit exponentials the kernel's weight of a
 * logit x <= 0 is table[E4M3(x)].  Asynchronous on `stream`.
 */
lamp_status lamp_exp8_table(uint8_t* table, void* stream);

/* Static name of a status code. */
const char* lamp_status_string(lamp_status s);

/* Detail of the last failing call on this thread ("" if none). */
const char* lamp_last_error(void);

/* LAMP_ABI_VERSION of the built library. */
int32_t lamp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LAMP_H_ */

/*
 * mla.h -- C ABI of the absorbed-latent MLA decode library for AMD MI355X (gfx950).
 *
 * Multi-head Latent Attention caches, per token and layer, a 512-wide latent
 * c_kv and a 64-wide decoupled RoPE key k_pe (576 elements, 1,152 B in bf16).
 * Decode folds each head's W_UK into its query, attends to the shared latent as
 * one "KV head" of width 576 (scores) / 512 (values), merges split partials with
 * a log-sum-exp combine, and expands the 512-wide result through W_UV.
 *
 * Sources cited below by key:
 *   [Audit]    "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界"
 *   [Report]   "DeepSeek-V2-Lite MLA 吸收式 KV 缓存优化 — 完整实验报告"
 *   [Tutorial] "手搓 MLA:从 MHA 到 weight absorption,看懂 DeepSeek 的 KV 压缩"
 *   [Budget]   "kv_budget.py" (TileLang tutorial, "算子实战 IV：MoE 与 MLA")
 *
 * Conventions shared by every call
 *   - All tensors are caller-owned device memory, passed as raw pointers; the
 *     library never allocates, frees or copies on the host's behalf, and never
 *     synchronises the stream.  Every call is asynchronous on `stream`
 *     (a hipStream_t; NULL is the default stream).  Inputs are never modified.
 *   - bf16 and fp16 tensors are passed as uint16_t bit patterns.
 *   - Device pointers must be 16-byte aligned (MLA_ERR_ALIGN otherwise).
 *   - Host-visible arguments are validated before anything is launched, so a
 *     call that returns an error has had no effect.  A failed launch returns
 *     MLA_ERR_HIP; mla_last_hip_error() then holds the hipError_t (per thread).
 *   - The first call that launches work checks that the current device is
 *     gfx950 and returns MLA_ERR_UNSUPPORTED otherwise.
 *   - Device-resident indices (slot_mapping, block_table, work items) cannot be
 *     checked on the host without a sync; kernels bounds-check them and skip
 *     what is out of range instead of faulting.
 *   - Calls on one stream are ordered; the library keeps no state between calls
 *     except the per-thread last HIP error and a per-device architecture flag.
 */
#ifndef MLA_ABSORBED_LATENT_H
#define MLA_ABSORBED_LATENT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL                         */
  MLA_ERR_SHAPE = 2,       /* unsupported head count / widths / block size        */
  MLA_ERR_VALUE = 3,       /* a size or scalar argument is out of range           */
  MLA_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned             */
  MLA_ERR_WORKSPACE = 5,   /* a caller buffer is too small (planner capacity)     */
  MLA_ERR_UNSUPPORTED = 6, /* the current device is not gfx950                    */
  MLA_ERR_HIP = 7          /* a HIP call or launch failed                         */
} mla_status;

/* Latent-cache formats ([Report] §3.2 and §4.1; the symmetric INT4, the
 * per-token INT8 and the FP8 variants are not ones the report measures; FP8
 * latent caches are named in [Audit] §6.1 and [Tutorial] §六 without a scaling
 * rule). */
typedef enum {
  MLA_CACHE_BF16 = 0,     /* c_kv and k_pe in bf16                                       */
  MLA_CACHE_INT8 = 1,     /* c_kv INT8, one fp32 scale per 32 channels; k_pe INT8 per 8   */
  MLA_CACHE_INT4 = 2,     /* c_kv asymmetric INT4, fp32 scale + zero per 32; k_pe INT8    */
  MLA_CACHE_INT4_SYM = 3, /* c_kv symmetric INT4, fp32 scale per 32; k_pe INT8            */
  MLA_CACHE_INT8_TOK = 4, /* c_kv INT8, one fp32 scale per token; k_pe INT8 per 8         */
  MLA_CACHE_FP8_TOK = 5,  /* c_kv e4m3 FP8, one fp32 scale per token; k_pe e4m3 per 8     */
  MLA_CACHE_INT4_SYM_K4 = 6, /* c_kv symmetric INT4 per 32; k_pe symmetric INT4 per 8      */
  MLA_CACHE_INT8_CHAN = 7   /* c_kv INT8, one fp32 scale per channel per 32-token block;
                               k_pe INT8 per 8 ([Report] §3.2 "per-channel INT8 (32 blocks)") */
} mla_cache_dtype;

/* Shape of one MLA layer.  Supported: num_heads in {16, 128}, qk_nope_dim = 128,
 * kv_lora_rank = 512, rope_dim = 64, v_head_dim = 128, block_size = 64; any
 * other value gives MLA_ERR_SHAPE.  softmax_scale must be finite and > 0
 * (1/sqrt(qk_nope_dim + rope_dim) for DeepSeek shapes). */
typedef struct {
  int32_t num_heads;
  int32_t qk_nope_dim;
  int32_t kv_lora_rank;
  int32_t rope_dim;
  int32_t v_head_dim;
  int32_t block_size;
  int32_t cache_dtype;   /* mla_cache_dtype */
  float softmax_scale;
} mla_config;

/* One unit of split-KV work: pages [first_page, first_page + n_pages) of
 * sequence `seq` (logical page numbers, i.e. indices into its block-table row);
 * the partial result is written to row `out_row` of o_part / lse_part.  The
 * range is clipped to the block-table row and to the sequence's length; an
 * item whose range is then empty (first_page past either) writes o = 0 and
 * lse = -inf.  An item with seq or out_row out of range, or a negative
 * first_page or n_pages, is skipped (its row is not written). */
typedef struct {
  int32_t seq;
  int32_t first_page;
  int32_t n_pages;
  int32_t out_row;
} mla_work_item;

/* ------------------------------------------------------------------ sizes
 * Pure host functions; they return 0 for an invalid config.
 * Bytes per token include every scale and zero point the decode reads:
 *   bf16 1,152 ([Audit] §2.4: 576 elements x 2 B), INT8 672, INT4 480,
 *   symmetric INT4 416, per-token INT8 612.
 * Page layouts (64 tokens, row = token):
 *   bf16: [64][576] bf16, latent in 0..511 then RoPE key in 512..575  (73,728 B)
 *   INT8: [64][576] int8 codes | [64][16] f32 latent scales
 *         | [64][8] f32 RoPE-key scales                               (43,008 B)
 *   INT4: [64][256] latent nibbles (element 2j in bits 0-3 of byte j, 2j+1 in
 *         bits 4-7) | [64][64] int8 RoPE-key codes | [64][16] f32 scales
 *         | [64][16] f32 zeros | [64][8] f32 RoPE-key scales          (30,720 B)
 *   INT4_SYM: as INT4 without the zeros; a nibble holds q + 8, q in -7..7
 *                                                                     (26,624 B)
 *   INT8_TOK: [64][576] int8 codes | [64] f32 latent scales
 *         | [64][8] f32 RoPE-key scales                               (39,168 B)
 *   FP8_TOK: as INT8_TOK with e4m3 codes                              (39,168 B)
 *   INT4_SYM_K4: [64][256] latent nibbles | [64][32] RoPE-key nibbles
 *         | [64][16] f32 scales | [64][8] f32 RoPE-key scales         (24,576 B)
 *   INT8_CHAN: [64][512] int8 latent codes | [64][64] int8 RoPE-key codes
 *         | [2][512] f32 channel scales (blocks 0, 1: tokens 0..31, 32..63)
 *         | [64][8] f32 RoPE-key scales | [32][512 B] overflow        (59,392 B)
 *         A block that has not yet received its 32nd token is "open": its
 *         latent rows are bf16, channels 0..255 of row r in code row
 *         32 b + r, channels 256..511 in overflow row r.  Bytes per token
 *         (672) count what the decode reads for a closed token.
 * A pool of N pages is N * mla_cache_page_bytes() contiguous bytes.          */
mla_status mla_config_check(const mla_config* cfg);
size_t mla_cache_bytes_per_token(const mla_config* cfg);
size_t mla_cache_page_bytes(const mla_config* cfg);
/* o_part (n_items x H x 512 fp16) plus lse_part (n_items x H f32), in bytes. */
size_t mla_decode_workspace_bytes(const mla_config* cfg, int32_t n_items);

/* ------------------------------------------------------------------ a-1
 * mla_cache_append: write n_tokens new cache rows into their pool slots.
 * [Audit] §2.4 and §4.1 (only the latent and the RoPE key are cached);
 * quantise-on-append for the INT8 / INT4 formats of [Report] §3.2.
 *   pool          device, num_pages * page_bytes, written
 *   c_kv          device [n_tokens][512] bf16 (post-RMSNorm latent)
 *   k_pe          device [n_tokens][64] bf16 (post-RoPE key)
 *   slot_mapping  device [n_tokens] int64, slot = page * 64 + offset; negative
 *                 or >= num_pages * 64 slots are skipped
 * INT8: per token, each group of 32 latent channels (8 for k_pe) gets
 *   scale = max|x| / 127 (IEEE fp32 division) and codes clamp(rint(x/scale),
 *   -127, 127) (round half to even); max|x| = 0 gives scale 0 and codes 0.
 * INT4: per group of 32 latent channels, zero = min, scale = (max-min)/15,
 *   q = clamp(rint((x-min)/scale), 0, 15); scale 0 gives q = 0.
 * INT8_TOK: as INT8 with one group of all 512 latent channels.
 * FP8_TOK: per token, scale = max|x| / 448 over the 512 latent channels (and
 *   over each 8-channel RoPE-key group); code = x / scale rounded to the
 *   nearest e4m3 value (OCP E4M3: bias 7, 3 mantissa bits, subnormals, no
 *   infinities), ties to even, saturating at +-448, sign bit of x / scale;
 *   max|x| = 0 gives scale 0 and codes 0.
 * INT4_SYM: per group of 32 latent channels, scale = max|x| / 7,
 *   q = clamp(rint(x/scale), -7, 7), stored as q + 8; max|x| = 0 gives scale 0
 *   and q = 0.  The RoPE key of INT4 and INT4_SYM is INT8 as above.
 * INT4_SYM_K4: INT4_SYM, and the RoPE key by the same rule in 8-channel groups.
 * INT8_CHAN: positions 32j..32j+31 of a sequence form a block; when the
 *   block's last position is appended, each latent channel c of the block gets
 *   scale = max_t |x[t][c]| / 127 and the INT8 codes above; earlier positions
 *   are stored as bf16 until then.  The RoPE key is INT8 per token as above.
 *   A call may hold several positions of a block only at consecutive indices
 *   in increasing slot order (as a prompt chunk or decode steps append them);
 *   a block whose rows were not all appended gets unspecified codes.  Two
 *   kernels run in order (block closing, then per-token work).
 * Codes and scales are bit-exact with that definition.
 * n_tokens == 0 is a no-op; n_tokens < 0 is MLA_ERR_VALUE.                  */
mla_status mla_cache_append(const mla_config* cfg, void* pool, int64_t num_pages,
                            const uint16_t* c_kv, const uint16_t* k_pe,
                            const int64_t* slot_mapping, int32_t n_tokens,
                            hipStream_t stream);

/* ------------------------------------------------------------------ a-2
 * mla_absorb_q: fold W_UK into the query ([Audit] §2.2; [Tutorial] §四,
 * einsum "thd,hdc->thc"):  q_abs[b,h,0:512] = sum_d q_nope[b,h,d] W_UK[h,d,:],
 * q_abs[b,h,512:576] = q_pe[b,h,:].
 *   q_nope  device [batch][H][128] bf16
 *   q_pe    device [batch][H][64]  bf16 (post-RoPE)
 *   w_uk    device [H][128][512]   bf16 (index order "hdc")
 *   q_abs   device [batch][H][576] fp16, written (fp32 accumulation, rounded
 *           to nearest even)
 * batch == 0 is a no-op.                                                   */
mla_status mla_absorb_q(const mla_config* cfg, const uint16_t* q_nope, const uint16_t* q_pe,
                        const uint16_t* w_uk, uint16_t* q_abs, int32_t batch,
                        hipStream_t stream);

/* ------------------------------------------------------------------ planner
 * mla_plan_splits: host-only, synchronous.  Cuts every sequence's pages into
 * contiguous runs of about `chunk_pages` pages (chunk_pages <= 0: chosen so the
 * whole batch makes at least ~num_cus work items), one work item per run.
 * A sequence with no tokens gets one empty item.  Items are ordered longest
 * first; out_row = split_offsets[seq] + (index of the run within its sequence).
 *   seq_lens_host      host [batch] int32, tokens per sequence (>= 0)
 *   items_host         host [max_items], written
 *   n_items            host, written
 *   split_offsets_host host [batch + 1], written (rows of sequence b are
 *                      split_offsets[b] .. split_offsets[b+1]-1)
 * MLA_ERR_WORKSPACE when max_items is too small (n_items then holds the
 * number needed).                                                          */
mla_status mla_plan_splits(const mla_config* cfg, const int32_t* seq_lens_host, int32_t batch,
                           int32_t num_cus, int32_t chunk_pages, mla_work_item* items_host,
                           int32_t max_items, int32_t* n_items, int32_t* split_offsets_host);

/* ------------------------------------------------------------------ a-3
 * mla_decode_attn: split-KV absorbed attention, MQA over the latent
 * ([Audit] §6.1: key width 576, value width 512; [Tutorial] §四).  For every
 * work item and head:
 *   s_t   = softmax_scale * (q_abs[b,h,0:512] . c_t + q_abs[b,h,512:576] . k_pe_t)
 *   o_j   = sum_t exp(s_t - m) c_t / sum_t exp(s_t - m),  m = max_t s_t
 *   lse_j = m + ln sum_t exp(s_t - m)             (natural log)
 * over the item's tokens t (a range of the sequence's first seq_lens[b] tokens).
 * An empty item gives lse_j = -inf and o_j = 0.  Quantised caches are
 * dequantised in registers (code * scale; q * scale + zero).  INT8_CHAN: the
 * closed blocks of the first floor(seq_lens[b] / 32) * 32 positions are read
 * as codes times their channel scales, the open block's rows as bf16; a
 * position that was never appended reads whatever the pool holds.
 *   q_abs        device [batch][H][576] fp16 (from mla_absorb_q)
 *   pool         device, num_pages pages in the config's format
 *   block_table  device [batch][max_pages_per_seq] int32 physical page ids;
 *                ids outside [0, num_pages) make their tokens contribute nothing;
 *                max_pages_per_seq <= 2^24 (MLA_ERR_VALUE otherwise)
 *   seq_lens     device [batch] int32
 *   items        device [n_items] (from mla_plan_splits, uploaded by the caller)
 *   o_part       device [n_items][H][512] fp16 (IEEE binary16 bits),
 *                lse_part device [n_items][H] f32
 *                (mla_decode_workspace_bytes(n_items) bytes in all); an item whose
 *                seq or out_row is out of range is skipped
 * Numerics: scores and probabilities use fp16 operands on the matrix cores
 * with fp32 accumulation; the bf16 latent is widened to fp16 exactly (values
 * beyond +-65504 are not supported); softmax state is fp32; the normalised
 * partial o_j is rounded to fp16 (round to nearest even), lse_j stays fp32.
 * Quantised caches are dequantised to fp16 with each fp32 scale (and INT4
 * zero point) rounded to fp16 first: the result stays within the output
 * tolerance while every group's scale is at least 2^-17 (INT8: max|x| of a
 * 32-channel group >= 127 * 2^-17, about 1e-3; INT4: max - min >= 15 * 2^-17),
 * including groups much smaller than the rest of their token; smaller scales
 * become fp16 subnormals and lose relative precision.  Zero points far above
 * their scale are fine: a dequantised value keeps fp16's relative precision.  */
mla_status mla_decode_attn(const mla_config* cfg, const uint16_t* q_abs, const void* pool,
                           int64_t num_pages, const int32_t* block_table,
                           int32_t max_pages_per_seq, const int32_t* seq_lens,
                           const mla_work_item* items, int32_t n_items,
                           uint16_t* o_part, float* lse_part, int32_t batch,
                           hipStream_t stream);

/* ------------------------------------------------------------------ a-4
 * mla_decode_combine: exact log-sum-exp merge of each sequence's partials:
 *   lse = ln sum_j exp(lse_j);  o_lat = sum_j exp(lse_j - lse) o_j.
 * A sequence whose partials are all empty gets o_lat = 0, lse = -inf.
 *   o_part, lse_part  as written by mla_decode_attn (fp16, f32); sums are fp32
 *   split_offsets  device [batch + 1] int32 (from mla_plan_splits)
 *   o_lat          device [batch][H][512] f32, written
 *   lse            device [batch][H] f32, written (may be NULL)            */
mla_status mla_decode_combine(const mla_config* cfg, const uint16_t* o_part, const float* lse_part,
                              const int32_t* split_offsets, float* o_lat, float* lse,
                              int32_t batch, hipStream_t stream);

/* ------------------------------------------------------------------ a-5
 * mla_out_proj: expand the latent result through W_UV ([Audit] §2.3;
 * [Tutorial] §四, einsum "thc,hdc->thd"):
 *   out[b,h,d] = sum_c W_UV[h,d,c] o_lat[b,h,c]            -> bf16
 * and optionally the layer output y[b,:] = W_O . concat_h(out[b,h,:]) -> bf16.
 *   o_lat      device [batch][H][512] f32
 *   w_uv       device [H][128][512] bf16 ("hdc")
 *   out        device [batch][H][128] bf16, written
 *   w_o        device [hidden][H*128] bf16 or NULL (then hidden, y and
 *              out_f32 are ignored)
 *   y          device [batch][hidden] bf16, written when w_o != NULL
 *   out_f32    device [batch][H][128] f32 workspace, required when w_o != NULL:
 *              receives `out` before its bf16 rounding; y is computed from it
 * The 512-wide operand is rounded to fp16 for the matrix cores (fp32 sums).  */
mla_status mla_out_proj(const mla_config* cfg, const float* o_lat, const uint16_t* w_uv,
                        uint16_t* out, const uint16_t* w_o, int32_t hidden, uint16_t* y,
                        float* out_f32, int32_t batch, hipStream_t stream);

/* ------------------------------------------------------------------ a-4 + a-5
 * mla_decode_combine_out_proj: mla_decode_combine followed by mla_out_proj in
 * one pass (same definitions and numerics: [Audit] §2.3; [Tutorial] §四):
 * o_lat is formed on chip from the partials and, unless asked for, never
 * written, which saves its round trip through HBM and a launch.
 *   o_part, lse_part, split_offsets   as for mla_decode_combine
 *   w_uv       device [H][128][512] bf16 ("hdc")
 *   out        device [batch][H][128] bf16, written
 *   o_lat      device [batch][H][512] f32, written when not NULL
 *   lse        device [batch][H] f32, written when not NULL
 *   w_o, hidden, y, out_f32   as for mla_out_proj (W_O product when w_o != NULL)
 * The merged o_lat enters the expansion rounded to fp16, as in mla_out_proj. */
mla_status mla_decode_combine_out_proj(const mla_config* cfg, const uint16_t* o_part, const float* lse_part,
                                       const int32_t* split_offsets, const uint16_t* w_uv, uint16_t* out,
                                       float* o_lat, float* lse, const uint16_t* w_o, int32_t hidden,
                                       uint16_t* y, float* out_f32, int32_t batch, hipStream_t stream);

/* ------------------------------------------------------------------ layer front
 * mla_layer_front: the projections that produce the hot path's inputs from a
 * layer's hidden states, V2-Lite form ([Report] §1.1: the joint down projection
 * yields the 512-wide latent and the 64-wide RoPE key; [Audit] §3.3: one query
 * projection, and the down projection's output puts the latent first;
 * [Tutorial] §三: the latent is RMS-normalised before caching, the RoPE key and
 * the query's RoPE part are rotated by position):
 *   q[t]   = W_q . x[t]                         (H x (128 + 64), head-major)
 *   kv[t]  = W_DKV . x[t]                       (512 + 64)
 *   c_kv[t] = kv[t][0:512] / sqrt(mean(kv[t][0:512]^2) + rms_eps)  (unit gain)
 *   k_pe[t] = RoPE(kv[t][512:576], positions[t])
 *   q_nope[t][h] = q[t][h][0:128],  q_pe[t][h] = RoPE(q[t][h][128:192], positions[t])
 * RoPE rotates the pairs (v[2i], v[2i+1]) by positions[t] * rope_base^(-2i/64).
 * Projections accumulate bf16 products in fp32 (on the matrix cores for 64
 * tokens or more with hidden a multiple of 64); the norm and the rotation run
 * in double precision; each output is rounded once to bf16 (round to nearest
 * even).
 *   x          device [n_tokens][hidden] bf16; hidden a positive multiple of 8
 *   w_q        device [H*192][hidden] bf16
 *   w_dkv      device [576][hidden] bf16
 *   positions  device [n_tokens] int32 (any value: used only as an angle)
 *   rms_eps    > 0;  rope_base > 1 (finite)
 *   workspace  device f32, >= mla_layer_front_workspace_bytes(cfg, n_tokens)
 *              bytes (given as workspace_bytes; MLA_ERR_WORKSPACE if smaller)
 *   q_nope     device [n_tokens][H][128] bf16, written
 *   q_pe       device [n_tokens][H][64] bf16, written
 *   c_kv       device [n_tokens][512] bf16, written
 *   k_pe       device [n_tokens][64] bf16, written
 * c_kv and k_pe are what mla_cache_append takes; q_nope and q_pe what
 * mla_absorb_q takes.  n_tokens == 0 is a no-op; n_tokens < 0 is
 * MLA_ERR_VALUE.  The library's output is independent of cfg->cache_dtype.  */
mla_status mla_layer_front(const mla_config* cfg, const uint16_t* x, int32_t hidden, const uint16_t* w_q,
                           const uint16_t* w_dkv, const int32_t* positions, float rms_eps, float rope_base,
                           float* workspace, size_t workspace_bytes, uint16_t* q_nope, uint16_t* q_pe,
                           uint16_t* c_kv, uint16_t* k_pe, int32_t n_tokens, hipStream_t stream);
/* n_tokens * (576 + H * 192) * 4 bytes: the fp32 projection results.        */
size_t mla_layer_front_workspace_bytes(const mla_config* cfg, int32_t n_tokens);

/* ------------------------------------------------------------------ layer front into the cache
 * mla_layer_front_append: mla_layer_front followed by
 * mla_cache_append(cfg, pool, num_pages, c_kv, k_pe, slot_mapping, n_tokens)
 * (same arguments, definitions and results, bit for bit: the cache rows are
 * written by the same row functions), with the append done by the launch that
 * normalises and rotates each token, so that the rows go into the cache without
 * a second pass over c_kv and k_pe: the fill path [Tutorial] §三 describes
 * (the latent normalised and the key rotated before they are cached).  c_kv and
 * k_pe are still written (mla_prefill_attn takes them).  The per-channel INT8
 * format is appended after the front by mla_cache_append's own two launches
 * (a block this call completes must be closed before the call's rows of the
 * next block take the page's overflow rows).
 *   pool, num_pages, slot_mapping  as for mla_cache_append (slots outside the
 *                                  pool are skipped)
 *   everything else                as for mla_layer_front
 * n_tokens == 0 is a no-op; n_tokens < 0 or num_pages < 0 is MLA_ERR_VALUE.   */
mla_status mla_layer_front_append(const mla_config* cfg, const uint16_t* x, int32_t hidden, const uint16_t* w_q,
                                  const uint16_t* w_dkv, const int32_t* positions, float rms_eps, float rope_base,
                                  float* workspace, size_t workspace_bytes, uint16_t* q_nope, uint16_t* q_pe,
                                  uint16_t* c_kv, uint16_t* k_pe, void* pool, int64_t num_pages,
                                  const int64_t* slot_mapping, int32_t n_tokens, hipStream_t stream);

/* ------------------------------------------------------------------ layer front, no allocation
 * mla_layer_front_noalloc: mla_layer_front (same arguments, definitions and
 * results, bit for bit) for callers that cannot allocate device memory --
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The fp32 projections live in a 16 MiB scratch array that the
 * library holds on every GPU it runs on until the process ends, instead of a
 * caller workspace; the call itself allocates nothing.
 *   n_tokens * (576 + H * 192) * 4 <= 16 MiB, i.e. n_tokens <= 1,149 (H = 16)
 *   or <= 166 (H = 128); larger n_tokens gives MLA_ERR_WORKSPACE.
 * All calls on one GPU share its scratch: calls that overlap on one GPU
 * (different streams, or host threads without ordering) race and must not be
 * issued.  The first call on a device looks up the scratch's device address
 * (no allocation); make it before capturing a graph.                        */
mla_status mla_layer_front_noalloc(const mla_config* cfg, const uint16_t* x, int32_t hidden, const uint16_t* w_q,
                                   const uint16_t* w_dkv, const int32_t* positions, float rms_eps, float rope_base,
                                   uint16_t* q_nope, uint16_t* q_pe, uint16_t* c_kv, uint16_t* k_pe,
                                   int32_t n_tokens, hipStream_t stream);

/* ------------------------------------------------------------------ residual
 * mla_out_residual: close a layer whose attention output is per head (as
 * mla_prefill_attn writes it): the output projection and the residual sum,
 *   x_out[t] = x_in[t] + W_O . concat_h(attn_out[t][h])     (fp32 sums) -> bf16
 * (W_O as in mla_out_proj; [Audit] §3.3 lists the output projection among a
 * V2-Lite layer's weights).  Stacked layers pass x_out on as the next layer's
 * hidden states.
 *   attn_out   device [n_tokens][H][128] bf16
 *   w_o        device [hidden][H*128] bf16
 *   x_in       device [n_tokens][hidden] bf16
 *   x_out      device [n_tokens][hidden] bf16, written; may be x_in
 *   workspace  device f32, >= n_tokens * hidden * 4 bytes (given as
 *              workspace_bytes; MLA_ERR_WORKSPACE if smaller)
 * hidden > 0; n_tokens == 0 is a no-op.  W_O runs on the matrix cores for
 * 64 tokens or more, else on the vector ALUs (one pass over its rows per 16
 * tokens); the sums are fp32 either way.                                     */
mla_status mla_out_residual(const mla_config* cfg, const uint16_t* attn_out, const uint16_t* w_o, int32_t hidden,
                            const uint16_t* x_in, uint16_t* x_out, float* workspace, size_t workspace_bytes,
                            int32_t n_tokens, hipStream_t stream);

/* ------------------------------------------------------------------ a-1 + a-2
 * mla_append_absorb_q: mla_cache_append followed by mla_absorb_q (same
 * arguments, definitions and results, bit for bit), in one launch when the
 * cache is bf16 (the append's copies run as extra work-groups of the absorb
 * kernel; the two touch disjoint memory).  Other formats launch the two
 * kernels in turn.  Either count may be 0.                                   */
mla_status mla_append_absorb_q(const mla_config* cfg, void* pool, int64_t num_pages, const uint16_t* c_kv,
                               const uint16_t* k_pe, const int64_t* slot_mapping, int32_t n_tokens,
                               const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_uk, uint16_t* q_abs,
                               int32_t batch, hipStream_t stream);

/* ------------------------------------------------------------------ prefill
 * mla_prefill_attn: causal attention of a chunk of T queries in the unabsorbed
 * form, the one engines use for prefill ([Tutorial] §四; the computation is
 * [Tutorial] §三's: each head's key and value rebuilt from the latent).  The
 * chunk is the last T of L positions of one sequence; query i sits at position
 * p_i = L - T + i and attends to positions 0..p_i:
 *   K_h[j] = [W_UK[h] c_j ; k_pe_j],  V_h[j] = W_UV[h] c_j,
 *   out[i][h] = sum_{j<=p_i} softmax_j(scale q_i,h . K_h[j]) V_h[j],
 *   lse[i][h] = ln sum_{j<=p_i} exp(scale q_i,h . K_h[j]).
 * K and V are formed in fp32 and kept in the workspace as fp16; the attention
 * products take fp16 operands (q widened exactly from bf16, P rounded) with
 * fp32 sums and softmax state.
 *   q_nope     device [T][H][128] bf16 (queries of positions L-T .. L-1)
 *   q_pe       device [T][H][64] bf16 (RoPE applied)
 *   n_queries  T, 0 <= T <= seq_len (0: no-op)
 *   c_kv, k_pe device [L][512], [L][64] bf16: every position of the sequence,
 *              the chunk's own included (as mla_layer_front writes them)
 *   seq_len    L, 1 <= L <= 2^23 (when T > 0)
 *   w_uk, w_uv device [H][128][512] bf16 ("hdc")
 *   workspace  device, >= mla_prefill_workspace_bytes(cfg, L) bytes (given as
 *              workspace_bytes; MLA_ERR_WORKSPACE if smaller)
 *   out        device [T][H][128] bf16, written
 *   lse        device [T][H] f32, written when not NULL
 * The result does not depend on cfg->cache_dtype (the latent comes in as bf16). */
mla_status mla_prefill_attn(const mla_config* cfg, const uint16_t* q_nope, const uint16_t* q_pe, int32_t n_queries,
                            const uint16_t* c_kv, const uint16_t* k_pe, int32_t seq_len, const uint16_t* w_uk,
                            const uint16_t* w_uv, void* workspace, size_t workspace_bytes, uint16_t* out,
                            float* lse, hipStream_t stream);
/* H * Lp * 512 bytes, Lp = seq_len rounded up to a multiple of 64.          */
size_t mla_prefill_workspace_bytes(const mla_config* cfg, int32_t seq_len);

/* ------------------------------------------------------------------ errors */
const char* mla_status_string(mla_status s);
int32_t mla_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_ABSORBED_LATENT_H */

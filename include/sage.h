/*
 * sage.h -- C ABI of the MI355X (gfx950) quantised-attention library (libsage.so).
 *
 * The library implements the forward hot path of SageAttention-style quantised
 * scaled-dot-product attention:
 *   K is smoothed by subtracting its per-channel mean over tokens; Q and K are
 *   quantised per block to INT8; S = Q K^T runs on INT8 matrix cores with INT32
 *   accumulation and is dequantised; an online (FlashAttention-style) softmax
 *   produces P, which is quantised to FP8 e4m3 (or kept in FP16/BF16) for the PV
 *   product, accumulated in two levels.
 * Sources: thu-ml/SageAttention repo card (vibecrowd.fund), "How it works"
 * (INT8 for QK^T, FP16/FP8 for PV, two-level PV accumulation); jisaku.com
 * glossary "SageAttention", 概要 and 主な特徴・仕組み (K smoothed along the
 * channel direction, P handled in FP8); heatdrop.ai review, "What it does" and
 * "The interesting bit" (drop-in for scaled_dot_product_attention, outlier
 * smoothing, two-level accumulation inside FP8 matrix units); cnnetsun.cn guide,
 * basic usage (q, k, v shaped (batch, heads, seq, head_dim), tensor_layout,
 * is_causal) and tuning tips (HND or NHD layout, causal masking).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.   Every tensor pointer is a DEVICE pointer (hipMalloc'd or from a
 *             framework allocator) on the current HIP device. The caller owns
 *             every buffer; the library allocates nothing, frees nothing and
 *             keeps no pointer after a call returns.
 * Stream.     `stream` is a hipStream_t passed as void* (NULL = the default
 *             stream). All work is enqueued asynchronously on it; no call
 *             synchronises. Calls on one stream are ordered; concurrent calls
 *             that share a workspace race.
 * Errors.     Arguments are validated on the host BEFORE any HIP call, and a
 *             non-SAGE_OK status means nothing was enqueued (SAGE_ERR_HIP aside:
 *             a launch that the runtime rejected). Faults inside kernels surface
 *             at the caller's next synchronisation. Nothing throws across the ABI.
 * Layouts.    Inputs/outputs use the caller's `layout`: HND = [B, H, N, d],
 *             NHD = [B, N, H, d], dense with d contiguous. Quantised codes and
 *             scales always use the canonical per-head orders given below.
 * Alignment.  Tensor and code pointers must be 16-byte aligned, scale/mean
 *             pointers 4-byte aligned (sage_attn_fwd_codes' v_scale: 16-byte),
 *             workspaces 256-byte aligned.
 * Aliasing.   No buffer a call writes (outputs, and the part of the workspace
 *             the size query reports) may overlap another such buffer or any
 *             buffer the call reads; that returns SAGE_ERR_INVALID_ARGUMENT.
 *             Read-only inputs may share memory (e.g. k == v).
 * Sizes.      1 <= B, Hq, Hkv; Hq % Hkv == 0 (group-query attention: query head
 *             h uses kv head h / (Hq/Hkv)); head_dim in {64, 128}; 0 <= Nq, Nk
 *             <= 2^20 (Nq == 0 or B == 0 is a valid no-op; Nk == 0 with Nq > 0
 *             is invalid: softmax over no keys).
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sage_status {
  SAGE_OK = 0,
  SAGE_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, bad enum, aliasing output */
  SAGE_ERR_UNSUPPORTED = 2,      /* valid request the library does not implement (head_dim, causal Nq != Nk) */
  SAGE_ERR_WORKSPACE = 3,        /* workspace smaller than the query function reports */
  SAGE_ERR_HIP = 4               /* the HIP runtime rejected a launch */
} sage_status;

typedef enum sage_layout { SAGE_LAYOUT_HND = 0, SAGE_LAYOUT_NHD = 1 } sage_layout;
typedef enum sage_dtype { SAGE_DTYPE_F16 = 0, SAGE_DTYPE_BF16 = 1 } sage_dtype;
/* PV product precision (repo card "How it works": FP16 or FP8 for PV).
 * SAGE_PV_FP16 keeps P and V in the input dtype (fp16, or bf16 for bf16 inputs). */
typedef enum sage_pv_dtype { SAGE_PV_FP16 = 0, SAGE_PV_FP8_E4M3 = 1 } sage_pv_dtype;
/* Granularity of the Q and K INT8 scales (heatdrop.ai review, "The interesting
 * bit": per-thread quantisation alongside the outlier smoothing).
 *   SAGE_QK_PER_BLOCK   BLK_Q = 128 query tokens and BLK_K = 64 key tokens per scale.
 *   SAGE_QK_PER_THREAD  one scale per group of tokens that a single lane of the
 *                       attention kernel's matrix instructions holds: every
 *                       query token alone (BLK_Q = 1) and every run of 16
 *                       consecutive keys (BLK_K = 16).
 * Zero is per-block, so a zero-initialised shape keeps the per-block scales. */
typedef enum sage_qk_gran { SAGE_QK_PER_BLOCK = 0, SAGE_QK_PER_THREAD = 1 } sage_qk_gran;

typedef struct sage_shape {
  int32_t batch;     /* B   */
  int32_t heads_q;   /* Hq  */
  int32_t heads_kv;  /* Hkv */
  int32_t seq_q;     /* Nq  */
  int32_t seq_k;     /* Nk  */
  int32_t head_dim;  /* d   */
  int32_t layout;    /* sage_layout of q, k, v and o */
  int32_t dtype;     /* sage_dtype of q, k, v and o  */
  int32_t qk_gran;   /* sage_qk_gran of the Q and K scales */
} sage_shape;

/* Quantisation block sizes and the online-softmax KV tile for `head_dim` and
 * the sage_qk_gran `qk_gran` (the blocks of the per-block INT8 quantisation:
 * thu-ml/SageAttention repo card, "How it works"; the per-thread groups:
 * heatdrop.ai review, "The interesting bit"). BLK_Q query tokens / BLK_K key tokens share one
 * INT8 scale (blocks start at token 0, the last one may be short); the softmax
 * walks KV tiles of BKV keys from key 0 upward, so BKV is part of the result's
 * definition (P's FP8 codes depend on the running row max).
 * Returns SAGE_ERR_UNSUPPORTED for other head dims, SAGE_ERR_INVALID_ARGUMENT
 * for an unknown granularity; null outputs are skipped. */
sage_status sage_block_sizes(int32_t head_dim, int32_t qk_gran, int32_t* blk_q, int32_t* blk_k, int32_t* bkv);

/* Nk rounded up to the padded key count of transposed V codes (a multiple of
 * BKV = 128): the row stride of the V operand of the FP8 (or FP16) PV product
 * (repo card, "How it works"). Returns 0 for seq_k <= 0. */
int64_t sage_v_codes_stride(int32_t seq_k);

/* Workspace bytes sage_quant_qk needs for `s` (K channel-sum partials of the
 * smoothing, jisaku.com glossary, 概要). 0 for an invalid shape. */
size_t sage_quant_qk_workspace_bytes(const sage_shape* s);
/* Workspace bytes sage_quant_v needs for `s` (V channel-absmax partials of the
 * FP8 V quantisation, repo card, "How it works"). 0 for an invalid shape. */
size_t sage_quant_v_workspace_bytes(const sage_shape* s);
/* Workspace bytes sage_attn_fwd needs for `s` and `pv` (all quantised
 * intermediates of the path the repo card's "How it works" describes: Q/K
 * codes and scales, K mean, V codes or transposed V, V scales, reduction
 * partials). Returns 0 for an invalid shape. */
size_t sage_workspace_bytes(const sage_shape* s, int32_t pv_dtype);

/* K smoothing + INT8 quantisation of Q and K, per block of s->qk_gran.
 * (glossary 概要: K smoothed along the channel direction, then INT8;
 *  repo card "How it works": INT8 for QK^T.)
 *   k_mean [B,Hkv,d] fp32      mu = fp32((sum over all Nk tokens, in fp64) / Nk).
 *              The fp64 sums are exact, so mu is the correctly rounded mean in
 *              every summation order, whenever no partial sum needs more than
 *              53 bits: for fp16 inputs when sum_t |k[t,c]| < 2^29 (for example
 *              |k| < 512 at Nk = 2^20); for bf16 inputs when sum_t |k[t,c]| <
 *              2^53 * g, g the finest unit in the last place among the
 *              channel's nonzero values. Beyond that the sum is deterministic
 *              and within an fp64 rounding of exact.
 *   q_codes [B,Hq,Nq,d] int8   round-half-even(fp32(q * fp32(127/a))), a = block absmax
 *   q_scale [B,Hq,ceil(Nq/BLK_Q)] fp32  a/127 (0 for an all-zero block, codes 0)
 *   k_codes [B,Hkv,Nk,d] int8  the same rule on fp32(k - mu)
 *   k_scale [B,Hkv,ceil(Nk/BLK_K)] fp32
 * Codes are in canonical HND order whatever `s->layout` is. */
sage_status sage_quant_qk(const sage_shape* s, const void* q, const void* k,
                          int8_t* q_codes, float* q_scale,
                          int8_t* k_codes, float* k_scale, float* k_mean,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Per-channel FP8 e4m3 (OCP, saturating, round-half-even) quantisation of V.
 * (repo card / heatdrop.ai "What it does": FP8 for the PV product.)
 *   v_scale [B,Hkv,d] fp32                       a_v/448, a_v = max over all tokens of |v|
 *   v_codes [B,Hkv,d,sage_v_codes_stride(Nk)] u8  e4m3(fp32(v * fp32(448/a_v))),
 *           keys contiguous per channel; padding keys are written as 0. */
sage_status sage_quant_v(const sage_shape* s, const void* v,
                         uint8_t* v_codes, float* v_scale,
                         void* workspace, size_t workspace_bytes, void* stream);

/* The whole forward: o = SageAttention(q, k, v), the call the pages show as
 * sageattn(q, k, v, tensor_layout="HND", is_causal=False) and as the drop-in
 * for scaled_dot_product_attention (cnnetsun.cn guide, basic usage; repo card,
 * "How to use"; heatdrop.ai review, "What it does").
 * is_causal: query i attends keys j <= i (top-left; requires Nq == Nk).
 * sm_scale:  softmax temperature (finite, > 0; 1/sqrt(d) for the drop-in).
 * pv_dtype:  sage_pv_dtype. o has q's shape, dtype and layout and must not
 *            overlap q, k, v or the workspace.
 * Runs, in order on `stream`: channel statistics, Q/K (and V) quantisation,
 * then the fused attention kernel (INT8 QK^T, dequantisation, online softmax,
 * P quantisation, PV with two-level accumulation, normalisation). */
sage_status sage_attn_fwd(const sage_shape* s, const void* q, const void* k, const void* v,
                          void* o, int32_t is_causal, float sm_scale, int32_t pv_dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Variable-length batches (heatdrop.ai review, "Key highlights": variable
 * sequence lengths within a batch). B sequences are packed along the token
 * axis: q [total_q, Hq, d], k and v [total_k, Hkv, d], o like q (the NHD order
 * of one long batch entry, dense, d contiguous). Sequence b owns the query
 * tokens [cu_seqlens_q[b], cu_seqlens_q[b+1]) and the key tokens
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]); both are DEVICE int32 arrays of B + 1
 * non-decreasing offsets from 0 to the total, and no sequence is longer than
 * its max_seqlen. Every sequence is one independent attention by the method:
 * its own K channel mean, Q/K INT8 blocks starting at its first token, its own
 * V channel scales, causal masking top-left within the sequence (query i sees
 * keys j <= i of its own sequence, also when its query and key counts differ).
 * A sequence with queries but no keys gets zero output rows.
 * The host never reads the device offsets. A table that breaks the rules above
 * gives unspecified output for the sequences involved, but every index is
 * clamped into the tensors and the workspace, so no access leaves them. */
typedef struct sage_varlen_shape {
  int32_t batch;         /* B sequences */
  int32_t heads_q;       /* Hq  */
  int32_t heads_kv;      /* Hkv */
  int32_t head_dim;      /* d   */
  int32_t total_q;       /* packed query tokens (= cu_seqlens_q[B]) */
  int32_t total_k;       /* packed key tokens (= cu_seqlens_k[B]) */
  int32_t max_seqlen_q;  /* bound on every sequence's query count, <= 2^20 */
  int32_t max_seqlen_k;  /* bound on every sequence's key count, <= 2^20 */
  int32_t dtype;         /* sage_dtype of q, k, v and o */
  int32_t qk_gran;       /* sage_qk_gran of the Q and K scales */
} sage_varlen_shape;

/* Workspace bytes sage_attn_fwd_varlen needs for `s` and `pv` (0 if invalid).
 * Sizes follow the totals and maximum lengths, not the device offsets. */
size_t sage_varlen_workspace_bytes(const sage_varlen_shape* s, int32_t pv_dtype);

/* The whole forward over a packed variable-length batch (see above); the other
 * arguments are as for sage_attn_fwd. Limits: 1 <= Hq, Hkv with Hq % Hkv == 0,
 * head_dim in {64, 128}, B * Hq <= 2^24, total_k + 127 * B <= 2^24 - 128 (the
 * padded key columns of the transposed V), (total_q / 256 + B) * Hq <= 2^30
 * (the attention work list). B == 0 or total_q == 0 is a no-op. With
 * total_k == 0 every output row is zero and k, v may be NULL.
 * cu_seqlens pointers must be 4-byte aligned; q, k, v, o 16-byte aligned. */
sage_status sage_attn_fwd_varlen(const sage_varlen_shape* s, const void* q, const void* k, const void* v,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* o,
                                 int32_t is_causal, float sm_scale, int32_t pv_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Workspace bytes sage_quant_varlen needs for `s` (the span table of the
 * sequences and the reduction partials). 0 for an invalid shape. */
size_t sage_quant_varlen_workspace_bytes(const sage_varlen_shape* s);

/* The quantisation stages of sage_attn_fwd_varlen on their own, per sequence
 * of a packed batch (heatdrop.ai review, "Key highlights": variable sequence
 * lengths within a batch; jisaku.com glossary, 概要, and the repo card's "How it
 * works" for the stages). Every sequence is quantised as a batch of one: its
 * own K channel mean, Q/K INT8 blocks from its first token, its own V channel
 * scales. Inputs and cu_seqlens as for sage_attn_fwd_varlen; outputs:
 *   q_codes    [Hq][total_q][d] int8     (sequence b: rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1)
 *   q_scale    [B][Hq][nbq] fp32         nbq = max(1, ceil(max_seqlen_q / BLK_Q)); sequence b writes
 *                                        its first ceil(nq_b / BLK_Q) entries
 *   k_codes    [Hkv][total_k][d] int8
 *   k_scale    [B][Hkv][nbk] fp32        nbk = max(1, ceil(max_seqlen_k / BLK_K)), likewise
 *   k_mean     [B][Hkv][d] fp32          0 for a sequence without keys
 *   v_prepared [Hkv][d][n_pad]           n_pad = 128 * ceil((total_k + 127 B) / 128), at least 128;
 *                                        FP8: e4m3 codes, FP16: the 16-bit values. Sequence b's keys
 *                                        are the columns p_b .. p_b + nk_b - 1, p_b = the sum over the
 *                                        earlier sequences of nk rounded up to 128; the columns up to
 *                                        p_b + nk_b rounded up to 128 hold zeros; others are not written
 *   v_scale    [B][Hkv][d] fp32          FP8 only: a_v / 448 per sequence and channel
 * pv_dtype selects the V stage. With total_q == 0 the Q outputs are not
 * written (q, q_codes, q_scale may be NULL); with total_k == 0 neither are the
 * K and V outputs (k, v and their outputs may be NULL). Alignment: tensors and
 * codes 16 bytes, scales, means and cu_seqlens 4 bytes, workspace 256 bytes. */
sage_status sage_quant_varlen(const sage_varlen_shape* s, int32_t pv_dtype, const void* q, const void* k,
                              const void* v, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int8_t* q_codes, float* q_scale, int8_t* k_codes, float* k_scale, float* k_mean,
                              void* v_prepared, float* v_scale, void* workspace, size_t workspace_bytes,
                              void* stream);

/* FP16-PV preparation of V (repo card, "How it works": FP16 for PV): the
 * 16-bit values transposed to
 *   v_t [B,Hkv,d,sage_v_codes_stride(Nk)] (keys contiguous per channel, padding keys 0),
 * the layout the PV product reads in FP16/BF16 mode. */
sage_status sage_transpose_v(const sage_shape* s, const void* v, void* v_t, void* stream);

/* Largest workspace sage_attn_fwd_noalloc can use: 32 MiB (for example
 * B = 1, 16 heads of 4096 tokens at head_dim 128). */
#define SAGE_NOALLOC_MAX_WORKSPACE_BYTES (32u * 1024u * 1024u)

/* sage_attn_fwd without a caller-supplied workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Arguments are as for sage_attn_fwd; the
 * caller still passes q, k, v and o. The workspace is a fixed device array of
 * SAGE_NOALLOC_MAX_WORKSPACE_BYTES inside the library, one per GPU, held until
 * the process ends; the call allocates and frees nothing (its first call on a
 * device looks the array's address up once). Errors: SAGE_ERR_WORKSPACE when
 * sage_workspace_bytes(s, pv_dtype) exceeds that limit, otherwise those of
 * sage_attn_fwd. Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams or threads) race and are not
 * allowed; calls on one stream are ordered and safe. Each call writes every
 * part of the array it later reads, so no state carries over between calls. */
sage_status sage_attn_fwd_noalloc(const sage_shape* s, const void* q, const void* k, const void* v,
                                  void* o, int32_t is_causal, float sm_scale, int32_t pv_dtype, void* stream);

/* The fused attention kernel alone, from precomputed codes: INT8 QK^T,
 * online softmax, P quantisation and two-level PV (repo card, "How it works";
 * jisaku.com glossary, 概要). For callers that quantise once and reuse K/V
 * codes, and to time the kernel by itself:
 *   q_codes/q_scale/k_codes/k_scale  as written by sage_quant_qk
 *   v_prepared  FP8: e4m3 codes from sage_quant_v;  FP16: v_t from sage_transpose_v
 *   v_scale     FP8: from sage_quant_v, 16-byte aligned (read four channels
 *               at a time);  FP16: ignored (may be NULL)
 * o, is_causal, sm_scale, pv_dtype as for sage_attn_fwd. Needs no workspace. */
sage_status sage_attn_fwd_codes(const sage_shape* s, const int8_t* q_codes, const float* q_scale,
                                const int8_t* k_codes, const float* k_scale, const void* v_prepared,
                                const float* v_scale, void* o, int32_t is_causal, float sm_scale,
                                int32_t pv_dtype, void* stream);

/* Test hook: the INT32 QK^T of the attention kernel's own matrix-core tile code
 * (the INT8 QK^T with INT32 accumulation of the repo card's "How it works"),
 * for canonical-order codes as produced by sage_quant_qk.
 *   s_out [B,Hq,Nq,Nk] int32, s_out[b,h,i,j] = sum_c q_codes[b,h,i,c] * k_codes[b,h/G,j,c]. */
sage_status sage_debug_qk_i32(const sage_shape* s, const int8_t* q_codes, const int8_t* k_codes,
                              int32_t* s_out, void* stream);

/* ---- FP4 microscaling variant (SageAttention3: heatdrop.ai review, "Key
 * highlights"; cnnetsun.cn guide, 序列长度优化技巧 -- named on the pages
 * without a format). Read as OCP MXFP4: FP4 E2M1 elements (values 0, 0.5, 1,
 * 1.5, 2, 3, 4, 6 and their negatives) with one E8M0 power-of-two scale byte
 * (2^(byte - 127)) per 32 elements along the contraction axis of each product.
 * The shared exponent of a block is floor(log2(max |x|)) - 2, clamped to
 * [-127, 127] (-127 for a block of zeros); each element is x / 2^exponent
 * rounded half to even, magnitudes above 6 saturating to 6. Codes are packed
 * two per byte, element 2i in the low nibble. K is smoothed by its channel mean
 * first, exactly as in sage_quant_qk (the same k_mean). Q is scaled before
 * its quantisation by c = fp32(sm_scale * log2 e) (sm_scale as passed, the
 * product in double, rounded once), so that the attention kernel's product
 * S2 = (Q c).K^T on the block-scaled FP4 matrix cores (fp32 sums) is already
 * in the log2 domain; then the online softmax over 128-key tiles, P~ to MXFP4 per query
 * row and 32 keys of the tile (the row sum adds the values that enter PV),
 * and PV with V in MXFP4, two-level accumulation, O / l in the epilogue.
 * s->qk_gran must be SAGE_QK_PER_BLOCK (0): the MX blocks are fixed; any
 * other valid value returns SAGE_ERR_UNSUPPORTED. */

/* Workspace bytes sage_quant_fp4 needs (K channel-sum partials, as for
 * sage_quant_qk). 0 for an invalid or unsupported shape. */
size_t sage_quant_fp4_workspace_bytes(const sage_shape* s);
/* Workspace bytes sage_attn_fwd_fp4 needs (all MXFP4 codes and scales, the K
 * mean and the partials). 0 for an invalid or unsupported shape. */
size_t sage_fp4_workspace_bytes(const sage_shape* s);

/* MXFP4 quantisation of Q (times c, see above), smoothed K and V, with
 * N = sage_v_codes_stride(Nk); sm_scale finite and > 0:
 *   q_codes [B,Hq,Nq,d/2] u8    q_scale [B,Hq,Nq,d/32] u8: fp32(q * c), blocks of 32 channels per token
 *   k_codes [B,Hkv,Nk,d/2] u8   k_scale [B,Hkv,Nk,d/32] u8: the same on fp32(k - k_mean)
 *   k_mean  [B,Hkv,d] fp32      as in sage_quant_qk
 *   v_codes [B,Hkv,d,N/2] u8    V transposed (keys contiguous per channel), blocks
 *                               of 32 keys from key 0; keys past Nk are code 0
 *   v_scale [B,Hkv,N/128,d,4] u8  per 128-key tile, each channel's four block
 *                               scales (16-byte aligned); blocks past Nk get 0
 * Codes are in canonical HND order whatever s->layout is. Skips Q when Nq == 0
 * and K/V when Nk == 0 (their pointers may then be NULL). */
sage_status sage_quant_fp4(const sage_shape* s, const void* q, const void* k, const void* v, float sm_scale,
                           uint8_t* q_codes, uint8_t* q_scale, uint8_t* k_codes, uint8_t* k_scale,
                           float* k_mean, uint8_t* v_codes, uint8_t* v_scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/* The FP4 attention kernel alone, from codes as sage_quant_fp4 writes them
 * (the softmax temperature is already in the Q codes); o and is_causal as for
 * sage_attn_fwd. Needs no workspace. The kernel reads k_scale in whole 4-byte
 * words: at d = 64 with B * Hkv * Nk odd, the buffer must stay readable for
 * the 2 bytes past its last scale byte (their values are not used). */
sage_status sage_attn_fwd_fp4_codes(const sage_shape* s, const uint8_t* q_codes, const uint8_t* q_scale,
                                    const uint8_t* k_codes, const uint8_t* k_scale, const uint8_t* v_codes,
                                    const uint8_t* v_scale, void* o, int32_t is_causal, void* stream);

/* The whole FP4 forward (quantisation then attention) on `stream`; arguments
 * and errors as for sage_attn_fwd without pv_dtype, the workspace sized by
 * sage_fp4_workspace_bytes. */
sage_status sage_attn_fwd_fp4(const sage_shape* s, const void* q, const void* k, const void* v, void* o,
                              int32_t is_causal, float sm_scale, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ---- The FP4 variant over a packed variable-length batch (heatdrop.ai
 * review, "Key highlights": variable sequence lengths within a batch, and the
 * FP4 microscaling variant above). Every sequence is quantised and attended
 * to as a batch of one: its own K channel mean, MX blocks of 32 channels per
 * token for Q and K, V blocks of 32 keys from the sequence's first key, causal
 * masking top-left within the sequence. Shape and cu_seqlens rules as for
 * sage_attn_fwd_varlen; s->qk_gran must be SAGE_QK_PER_BLOCK (0), any other
 * valid value returns SAGE_ERR_UNSUPPORTED. */

/* Workspace bytes sage_attn_fwd_fp4_varlen needs (span table, work list, all
 * MXFP4 codes and scales, the K means, the partials); 0 for an invalid or
 * unsupported shape. */
size_t sage_fp4_varlen_workspace_bytes(const sage_varlen_shape* s);

/* The whole FP4 forward over a packed batch: q [total_q, Hq, d], k and v
 * [total_k, Hkv, d], o [total_q, Hq, d] (s->dtype), is_causal 0 or 1, sm_scale
 * finite and > 0. B == 0 or total_q == 0 is a no-op; with total_k == 0 every
 * output row is zero and k, v may be NULL. Alignment as for
 * sage_attn_fwd_varlen. */
sage_status sage_attn_fwd_fp4_varlen(const sage_varlen_shape* s, const void* q, const void* k, const void* v,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* o,
                                     int32_t is_causal, float sm_scale, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Workspace bytes sage_quant_fp4_varlen needs (span table, work list and the
 * K channel-sum partials); 0 for an invalid or unsupported shape. */
size_t sage_quant_fp4_varlen_workspace_bytes(const sage_varlen_shape* s);

/* The MXFP4 stages of sage_attn_fwd_fp4_varlen on their own. Outputs, with
 * n_pad as for sage_quant_varlen and sequence b's key columns from p_b there:
 *   q_codes [Hq][total_q][d/2] u8    q_scale [Hq][total_q][d/32] u8 (Q times c, as in sage_quant_fp4)
 *   k_codes [Hkv][total_k][d/2] u8   k_scale [Hkv][total_k][d/32] u8 (K minus its sequence's mean)
 *   k_mean  [B][Hkv][d] fp32         0 for a sequence without keys
 *   v_codes [Hkv][d][n_pad/2] u8     V transposed; the columns p_b .. p_b + nk_b rounded up to 128
 *                                    hold sequence b (keys past nk_b are code 0), others are not written
 *   v_scale [Hkv][n_pad/128][d][4] u8  per 128-column tile, each channel's four block scales (blocks
 *                                    past nk_b get 0), the tiles of sequence b as for v_codes
 * With total_q == 0 the Q outputs are not written (q and they may be NULL);
 * with total_k == 0 neither are the K and V outputs. Alignment: tensors and
 * codes 16 bytes (v_scale too), scales, means and cu_seqlens 4 bytes,
 * workspace 256 bytes. */
sage_status sage_quant_fp4_varlen(const sage_varlen_shape* s, const void* q, const void* k, const void* v,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, float sm_scale,
                                  uint8_t* q_codes, uint8_t* q_scale, uint8_t* k_codes, uint8_t* k_scale,
                                  float* k_mean, uint8_t* v_codes, uint8_t* v_scale, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Static description of a status code (never NULL). Part of the error
 * convention above, not of the method. */
const char* sage_status_string(sage_status st);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_H */

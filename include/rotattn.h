/*
 * rotattn: RoPE-aware-rotated mixed-precision INT4 FlashAttention for
 * video-DiT self-attention with 3D RoPE, for AMD Instinct MI355X (gfx950).
 *
 * The method is the one the RotateAttention abstract (arXiv 2607.02584)
 * describes: 3D RoPE on Q and K, an orthonormal Walsh-Hadamard rotation
 * applied after RoPE (the variant of its RoPE-aware rotation that runs online
 * at little cost), symmetric INT4 Q/K/V, a fused flash loop with integer Q.K^T,
 * float32 online softmax and the range-optimized P quantization (fixed scale
 * 1/15, zero-point -8), and an FP16 path for the blocks, heads and denoising
 * steps where INT4 would lose too much accuracy. The flash loop follows the online-softmax
 * recurrences and the block mask of RainFusion2.0, section 3.1 "Blockwise
 * Sparse".
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are device (HBM) addresses that the caller
 *    allocates and owns. The library never allocates or frees memory; all
 *    scratch lives in the caller's workspace (size from
 *    rotattn_workspace_bytes), except for rotattn_quantize_qk_static, which
 *    uses a static device buffer of the library (see there).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream). No call synchronizes with the host. A call enqueues kernels
 *    and event records only (no memsets or copies), so it can be captured in
 *    a HIP graph; the calls that can route rows to FP16 fork a library-owned
 *    side stream from `stream` with an event and join it back before they
 *    return, so all of their work is ordered before later work on `stream`.
 *  - Return ROTATTN_OK (0) on success or a negative ROTATTN_E* code.
 *    Argument errors are detected on the host before anything is enqueued
 *    and leave every output untouched. ROTATTN_ELAUNCH reports a failed
 *    kernel launch (from hipGetLastError); outputs are then undefined.
 *  - Inputs are not checked for NaN or Inf.
 *  - Attention is non-causal (video-DiT self-attention).
 *
 * Shapes: B batch, H heads, L tokens, D head dim (64 or 128). Tokens are the
 * text prefix (no RoPE) followed by the video latent grid grid_t x grid_h x
 * grid_w flattened frame-major, the default [F, H, W] order of RainFusion2.0
 * ("3D Window Permutation"). Lp = L rounded up to a multiple of 64,
 * NB = Lp / 64, D' = D for ROTATTN_ROT_FULL and ROTATTN_ROT_PAIR, 192 for
 * ROTATTN_ROT_GROUP64.
 */
#ifndef ROTATTN_H
#define ROTATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROTATTN_VERSION 5

/* error codes */
#define ROTATTN_OK            0
#define ROTATTN_EINVAL       -1  /* null pointer, bad size, split or stride */
#define ROTATTN_EUNSUPPORTED -2  /* head dim other than 64 or 128; a RoPE group wider than 64 with ROT_GROUP64;
                                    L > 2^30, H > 65535, 2B > 65535 or B*H*NB >= 2^24 (launch limits); RoPE
                                    tables of 2^31 floats or more (sum over axes of 2 * grid size * pairs) */
#define ROTATTN_EALIGN       -3  /* a pointer or row stride not 16-byte aligned */
#define ROTATTN_EWORKSPACE   -4  /* workspace missing or smaller than rotattn_workspace_bytes */
#define ROTATTN_ELAUNCH      -5  /* a kernel launch failed */
#define ROTATTN_ESCRATCH     -6  /* more scratch needed than rotattn_quantize_qk_static's static buffer holds */

/* rotation applied after RoPE (RotateAttention abstract, "RoPE-aware Rotation") */
#define ROTATTN_ROT_FULL    0  /* x' = x H_D / sqrt(D) over the whole head dim; D' = D */
#define ROTATTN_ROT_GROUP64 1  /* each RoPE group zero padded to 64 and turned by H_64 / 8; D' = 192 */
#define ROTATTN_ROT_PAIR    2  /* the mergeable rotation: every RoPE pair (2i, 2i+1) turned by pi/4 in its own
                                  plane, folded into RoPE (video tokens: angle pos * theta_i + pi/4; text tokens:
                                  pi/4); it commutes with every RoPE rotation; D' = D */

/* calls, for rotattn_workspace_bytes */
#define ROTATTN_CALL_QUANTIZE_QK 0
#define ROTATTN_CALL_QUANTIZE_V  1
#define ROTATTN_CALL_ATTENTION   2
#define ROTATTN_CALL_FORWARD     3
#define ROTATTN_CALL_FP16_FORWARD 4
#define ROTATTN_CALL_DEBUG_DUMP  5
#define ROTATTN_CALL_BLOCK_MASK  6
#define ROTATTN_CALL_SPARSE_ATTENTION 7
#define ROTATTN_CALL_ATTENTION_HEAD_FALLBACK 8  /* rotattn_attention with a head_fallback mask */
#define ROTATTN_CALL_FORWARD_HEAD_FALLBACK   9  /* rotattn_forward with a head_fallback mask */

typedef void* rotattn_stream_t; /* hipStream_t */

/* Problem description, passed by pointer to every call (host memory, read only). */
typedef struct rotattn_problem {
  int32_t B, H, L, D;
  int32_t grid_t, grid_h, grid_w;  /* video latent grid; L = text_prefix + grid_t*grid_h*grid_w */
  int32_t text_prefix;             /* leading text tokens that take no RoPE */
  int32_t rope_split[3];           /* head dims of the t, h, w RoPE groups, contiguous, sum = D */
  int32_t rotation;                /* ROTATTN_ROT_FULL, ROTATTN_ROT_GROUP64 or ROTATTN_ROT_PAIR */
  double rope_base;                /* RoPE frequency base (10000) */
  int64_t stride_b, stride_h, stride_l; /* element strides of q, k, v and out; the D axis is contiguous */
  float block_err_tau;             /* a Q/K block whose quantization NSR exceeds this runs on FP16; +inf: never */
  int32_t reserved;
} rotattn_problem;

/* Outputs of rotattn_quantize_qk, inputs of rotattn_attention / rotattn_forward. All device. */
typedef struct rotattn_qk_buffers {
  uint8_t* q_codes;     /* [B][H][Lp][D'/2]: byte k = dim 2k (low nibble) | dim 2k+1 (high nibble), two's complement INT4 */
  uint8_t* k_codes;     /* same layout */
  float* q_scale;       /* [B][H][NB] per-64-token-block scale s = absmax/7 */
  float* k_scale;
  uint8_t* q_flag;      /* [B][H][NB] 1 if the block's quantization NSR > block_err_tau */
  uint8_t* k_flag;
  uint32_t* head_kflag; /* [B*H] number of flagged K blocks of the head (nonzero if any is flagged) */
  void* q_rope;         /* optional fp16 [B][H][L][D] (dense): RoPE'd, unrotated Q for the FP16 path (with
                           ROTATTN_ROT_PAIR the pair rotation is part of RoPE and included); NULL = not written */
  void* k_rope;         /* optional, as q_rope */
  float* q_bsum;        /* optional float [B][H][NB][D] (16-byte aligned): per 64-token block, the sum of the RoPE'd,
                           unrotated rows over the block's valid tokens (float32, ascending token order); the input
                           of rotattn_block_mask; NULL = not written */
  float* k_bsum;        /* optional, as q_bsum */
} rotattn_qk_buffers;

/* Quantized V. All device. */
typedef struct rotattn_v_buffers {
  uint8_t* v_codes;  /* [B][H][NB][D][32]: the 64 keys of one block and channel, nibble packed in the order the
                        INT4 kernel's matrix-core operands use: byte 16*hh + 8*s + 4*w + b holds, in its low
                        nibble, the code of key 32*s + 16*w + 4*hh + b and, in its high nibble, the code of key
                        32*s + 16*w + 8 + 4*hh + b (hh, s, w in {0,1}, b in 0..3) */
  float* v_scale;    /* [B][H][D] per-channel scale s_v = absmax over the L tokens / 7 */
  int32_t* v_colsum; /* [B][H][NB][D] integer sum of the 64 codes of each key block and channel */
} rotattn_v_buffers;

/* Buffer sizes in bytes for a problem (host only, no device work). */
typedef struct rotattn_sizes {
  int64_t Lp, NB, Dp;
  int64_t qk_codes_bytes;  /* each of q_codes, k_codes */
  int64_t qk_scale_bytes;  /* each of q_scale, k_scale */
  int64_t qk_flag_bytes;   /* each of q_flag, k_flag */
  int64_t head_flag_bytes; /* head_kflag */
  int64_t rope_bytes;      /* each of q_rope, k_rope */
  int64_t v_codes_bytes, v_scale_bytes, v_colsum_bytes;
  int64_t out_min_elems;   /* smallest element count an output buffer with the problem's strides spans */
  int64_t bsum_bytes;      /* each of q_bsum, k_bsum */
  int64_t mask_rows;       /* 128-row query blocks of a block-sparse mask: ceil(NB / 2) */
  int64_t mask_words;      /* uint32 words per mask row: ceil(NB / 32) */
  int64_t mask_bytes;      /* block-sparse mask [B][H][mask_rows][mask_words] uint32 */
} rotattn_sizes;

/* Library version (ROTATTN_VERSION). */
int rotattn_version(void);

/* Static message for an error code; never NULL. */
const char* rotattn_strerror(int code);

/* Validate `p` and fill `out` with the buffer sizes. Errors: EINVAL, EUNSUPPORTED. */
int rotattn_get_sizes(const rotattn_problem* p, rotattn_sizes* out);

/* Workspace bytes that call `call` (ROTATTN_CALL_*) needs for `p`. Errors: EINVAL, EUNSUPPORTED. */
int rotattn_workspace_bytes(const rotattn_problem* p, int call, size_t* bytes);

/*
 * Steps 1-3 for Q and K (RotateAttention abstract): 3D RoPE (float32, each
 * pair turned by pos * base^(-2i/g_rot) of its axis group), the RoPE-aware
 * rotation (the Walsh-Hadamard after RoPE, or with ROTATTN_ROT_PAIR the pair
 * rotation folded into RoPE), symmetric INT4 quantization per 64-token block
 * (s = absmax/7, codes clamp(rne(x/s), -7, 7)) and the block error flags
 * (NSR = |x - s c|^2 / |x|^2 > block_err_tau); optionally the RoPE'd block
 * sums of block-sparse attention (out->q_bsum, out->k_bsum).
 * q, k: device fp16 with the problem's strides, 16-byte aligned rows.
 * out: codes, scales, flags, head_kflag (all required); q_rope/k_rope
 * optional (required later by rotattn_attention when FP16 fallback can occur).
 * Workspace: ROTATTN_CALL_QUANTIZE_QK bytes. After the call it holds the RoPE
 * tables the prologue used, from byte 0: for each axis t, h, w in turn,
 * float32 cos[n_pos][npair] followed by sin[n_pos][npair] (n_pos the grid
 * size of the axis, npair = rope_split / 2 rounded down), each value
 * cos/sin(pos * base^(-2i / (2 npair)) (+ pi/4 with ROTATTN_ROT_PAIR))
 * evaluated in double and rounded once to float.
 */
int rotattn_quantize_qk(const rotattn_problem* p, const void* q, const void* k,
                        const rotattn_qk_buffers* out, void* workspace, size_t workspace_bytes,
                        rotattn_stream_t stream);

/*
 * rotattn_quantize_qk without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Same arguments, outputs and errors as
 * rotattn_quantize_qk; its scratch (the RoPE tables) lives in a static
 * 1 MiB device array of the library, one copy per device, held until the
 * process ends. Problems whose tables need more than 1 MiB (see
 * rotattn_workspace_bytes(ROTATTN_CALL_QUANTIZE_QK)) return ROTATTN_ESCRATCH
 * before anything is enqueued. The stream must belong to the device current
 * on the calling thread (else ROTATTN_EINVAL). Calls share their device's
 * array: calls that overlap on one device (different streams, or threads
 * without ordering between them) race on it. It calls no allocating routine.
 */
int rotattn_quantize_qk_static(const rotattn_problem* p, const void* q, const void* k,
                               const rotattn_qk_buffers* out, rotattn_stream_t stream);

/*
 * Per-channel symmetric INT4 quantization of V over all L tokens of a head,
 * with per-64-key-block column sums (the zero-point correction term of the
 * P.V product). v: device fp16 with the problem's strides.
 * Workspace: ROTATTN_CALL_QUANTIZE_V bytes.
 */
int rotattn_quantize_v(const rotattn_problem* p, const void* v, const rotattn_v_buffers* out,
                       void* workspace, size_t workspace_bytes, rotattn_stream_t stream);

/*
 * Step 4 and the FP16 fallback, from quantized inputs: the fused INT4 flash
 * loop (RainFusion2.0 sec. 3.1 recurrences in the log2 domain) with integer
 * Q.K^T on the matrix cores, float32 online softmax, P codes
 * pq = rne(15 P) - 8, and integer P.V against the per-channel V codes with
 * the 8 * column-sum zero-point correction; output
 * out = O * (s_v / 15) / l in fp16.
 * Routing (selective FP16 fallback): tile (query block i, key block j) runs
 * on the FP16 path when head_fallback[b*H+h] != 0, or q_flag[i], or
 * k_flag[j]. A query block that mixes both paths runs its INT4 tiles first
 * (their running max, and so their P codes, see the INT4 tiles only); its
 * FP16 tiles then continue the same online softmax (in a head with at most
 * 16 flagged K blocks), or run as a partial result of their own merged with
 * the INT4 one (more than 16): either is the log-sum-exp merge of the two
 * partial results.
 * head_fallback: device uint8 [B*H] or NULL (no head is masked). When it is
 * non-NULL or block_err_tau is finite, qk->q_rope and qk->k_rope and v are
 * required (the FP16 path reads them); otherwise they may be NULL.
 * out: device fp16 with the problem's strides (may not alias inputs).
 * Workspace: ROTATTN_CALL_ATTENTION bytes without a head mask,
 * ROTATTN_CALL_ATTENTION_HEAD_FALLBACK bytes with one: the K/V block images
 * the INT4 kernel copies into LDS (1.5x the packed K + V codes at
 * D' = D = 128); when the FP16 path can run (a head mask, or
 * block_err_tau finite), the transposed fp16 V blocks it reads (L x D fp16
 * rounded up to whole blocks); with block_err_tau finite, room for the INT4
 * partial results of rows that mix both paths (float32 O, m, l per row).
 */
int rotattn_attention(const rotattn_problem* p, const rotattn_qk_buffers* qk, const rotattn_v_buffers* vq,
                      const void* v, const uint8_t* head_fallback, void* out,
                      void* workspace, size_t workspace_bytes, rotattn_stream_t stream);

/*
 * rotattn_quantize_v into the workspace followed by rotattn_attention: the
 * whole attention call after rotattn_quantize_qk (steps 3 for V and 4 of the
 * RotateAttention abstract's path, with its selective FP16 fallback).
 * Workspace: ROTATTN_CALL_FORWARD bytes without a head mask,
 * ROTATTN_CALL_FORWARD_HEAD_FALLBACK bytes with one.
 */
int rotattn_forward(const rotattn_problem* p, const rotattn_qk_buffers* qk, const void* v,
                    const uint8_t* head_fallback, void* out,
                    void* workspace, size_t workspace_bytes, rotattn_stream_t stream);

/*
 * Whole-call FP16 flash attention with 3D RoPE, no rotation or quantization:
 * the fallback for a whole denoising step (RotateAttention abstract).
 * Workspace: ROTATTN_CALL_FP16_FORWARD bytes (RoPE tables, RoPE'd copies of
 * Q and K, transposed V blocks).
 */
int rotattn_fp16_forward(const rotattn_problem* p, const void* q, const void* k, const void* v, void* out,
                         void* workspace, size_t workspace_bytes, rotattn_stream_t stream);

/*
 * Test hook: runs the INT4 flash kernel, instantiated with its dump switch,
 * on selected 64-row query blocks and writes its intermediate integers.
 * units: device int32 [n_units], unit = (b*H + h)*NB + query_block.
 * Outputs (device, caller zero-fills; blocks skipped by routing stay untouched):
 *   acc_qk  int32 [n_units][64][Lp]   integer q.k over the rotated dims
 *   p_codes int8  [n_units][64][Lp]   pq in [-8, 7]
 *   acc_pv  int32 [n_units][64][NB][D] sum over the block of (pq + 8) * v_code
 *                                      (= pq . v + 8 * colsum)
 *   m_hist  float [n_units][64][NB]   running max (log2 domain) after each block
 *   p15     float [n_units][64][Lp]   the float32 value 15 P that each P code is rounded from
 *                                      (optional: NULL = not written)
 * Rows at or beyond L are not written. head_fallback as in rotattn_attention.
 * block_mask: NULL (dense) or a block-sparse mask as in
 * rotattn_sparse_attention (then head_fallback must be NULL and
 * block_err_tau +inf; key blocks the mask drops stay untouched).
 * Workspace: ROTATTN_CALL_DEBUG_DUMP bytes (the K/V block images).
 */
int rotattn_debug_dump(const rotattn_problem* p, const rotattn_qk_buffers* qk, const rotattn_v_buffers* vq,
                       const uint8_t* head_fallback, const uint32_t* block_mask, const int32_t* units,
                       int32_t n_units,
                       int32_t* acc_qk, int8_t* p_codes, int32_t* acc_pv, float* m_hist, float* p15,
                       void* workspace, size_t workspace_bytes, rotattn_stream_t stream);

/*
 * Block mask of block-sparse attention (RainFusion2.0, sec. 3.2
 * "Representative Token for Blocks" and sec. 3.4 "First Frame Sink").
 * Query blocks of 128 rows, key blocks of 64 keys (sec. 3.1 lets the two
 * block sizes differ; 128 rows are one workgroup of the INT4 kernel).
 * Representative tokens: the mean of every block of the RoPE'd (unrotated) Q
 * and K over the block's valid tokens, from the block sums rotattn_quantize_qk
 * writes into qk->q_bsum / qk->k_bsum (a 128-row query block adds its two
 * sums; each sum is divided by its row count in float32). For query block i,
 * S_hat[i][j] = q_hat_i . k_hat_j (one float32 fma chain over the head dim);
 * the topn key blocks with the largest S_hat are kept (equal scores: lower j
 * first), then every key block holding a text-prefix or first-frame token
 * (tokens below text_prefix + grid_h * grid_w) is kept, and a query block
 * holding such a token keeps every key block.
 * qk: the buffers of rotattn_quantize_qk; only q_bsum and k_bsum are read
 * (required).
 * topn >= 1 (topn >= NB keeps everything).
 * mask: device uint32 [B][H][mask_rows][mask_words] (rotattn_sizes), 4-byte
 *   aligned: bit (j % 32) of word j / 32 of row (b, h, i) = 1 iff key block j
 *   is kept for query rows [128 i, 128 i + 128); bits at or beyond NB are 0.
 * Errors: EINVAL (null pointer, topn < 1), EUNSUPPORTED (NB > 16384 or
 * B*H > 65535), EALIGN.
 * Workspace: none (ROTATTN_CALL_BLOCK_MASK is 0 bytes; NULL is accepted).
 */
int rotattn_block_mask(const rotattn_problem* p, const rotattn_qk_buffers* qk, int32_t topn, uint32_t* mask,
                       void* workspace, size_t workspace_bytes, rotattn_stream_t stream);

/*
 * Block-sparse INT4 attention (RainFusion2.0, sec. 3.1 "Blockwise Sparse":
 * Q_i K_j^T and P_ij V_j are skipped where M_ij = 0): the INT4 flash loop of
 * rotattn_attention over the key blocks the mask keeps for each query block,
 * in ascending order. block_mask as written by rotattn_block_mask (any mask
 * of that layout is accepted; a query block that keeps no key block gets
 * zeros). Block routing does not combine with it: block_err_tau must be
 * +inf (else EINVAL); there is no FP16 fallback on this call.
 * out: device fp16 with the problem's strides.
 * Workspace: ROTATTN_CALL_SPARSE_ATTENTION bytes (the K/V block images).
 */
int rotattn_sparse_attention(const rotattn_problem* p, const rotattn_qk_buffers* qk, const rotattn_v_buffers* vq,
                             const uint32_t* block_mask, void* out, void* workspace, size_t workspace_bytes,
                             rotattn_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ROTATTN_H */

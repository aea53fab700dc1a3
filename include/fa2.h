/*
 * fa2.h -- C ABI of the MI355X (gfx950) FlashAttention-2 forward library.
 *
 * Operation (the page "CuTe 详解：以 FlashAttention-2 拆解 Layout、TiledCopy 与
 * TiledMMA", §"先看全局：FA2 中的数据究竟去了哪里" and §"教学配置：一块 CTA 做什么"):
 * for every batch b, head h and query row i,
 *     s_ij  = scale * q_i . k_j           for admissible keys j
 *     O_i   = sum_j softmax_j(s_i) v_j
 *     LSE_i = log(sum_j exp(s_ij))        (natural log)
 * where the admissible keys are 0..S-1, or 0..i when `causal` is set. It is
 * computed tile by tile with an online softmax (§"沿 C fragment 做 Online
 * Softmax"), so no S x S matrix is ever stored; the result equals the plain
 * definition up to floating-point rounding. O and the log-sum-exp are the
 * outputs the page lists for the production kernel (§"与官方 FA2 比较时，先对齐
 * 契约"); tensors are [B,H,N,D] row-major as there.
 *
 * fa2_fwd_ex and fa2_fwd_varlen add the features the same page lists for a
 * production FA2 (§"哪些结论可以迁移，哪些只是本例特例": local masks, variable
 * length sequences, dropout, GQA/MQA). The page names them without defining
 * them; the definitions below are the plain readings used throughout this
 * library:
 *   GQA/MQA  H query heads share H_kv K/V heads (H a multiple of H_kv): query
 *            head h reads K/V head h / (H / H_kv). H_kv = 1 is MQA.
 *   window   key j is admissible for query i when
 *            i - window_left <= j <= i + window_right; a side given as -1 is
 *            unbounded. (-1, -1) admits every key, (-1, 0) is causal.
 *   varlen   several sequences packed along the row axis; each attends only
 *            within itself (queries and keys of one sequence, row indices
 *            counted from the sequence start).
 *   dropout  after the softmax, each probability P_ij is kept with
 *            probability 1 - p and scaled by 1/(1 - p), else set to 0:
 *            O_i = sum_j P_ij z_ij v_j / (1 - p). LSE is that of the softmax
 *            before dropout. z_ij comes from Philox4x32-10 (Salmon et al.,
 *            SC 2011, "Parallel random numbers: as easy as 1, 2, 3"): with
 *            r = Philox4x32-10(counter = (j / 8, i, b*H + h, offset),
 *                              key = (seed mod 2^32, seed / 2^32))
 *            read as eight 16-bit draws (draw t = bits 16*(t mod 2) .. +15 of
 *            word t / 2), z_ij = 1 when draw j mod 8 is >= floor(p * 2^16)
 *            (clamped to 2^16 - 1), where i and j are row indices within the
 *            sequence and b is the batch index (the sequence index when
 *            packed). The keep probability is therefore 1 - floor(p*2^16)/2^16,
 *            within 2^-16 of 1 - p.
 *
 * Precision: fp16 inputs, fp32 accumulation (MFMA), fp32 softmax state, fp16
 * output rounded to nearest even, fp32 LSE.
 *
 * Inputs must be finite. With an infinity or NaN among q, k or v the call still
 * completes and writes every output, but the values are unspecified (the
 * kernel's max and overflow tests assume finite scores).
 */
#ifndef FA2_H
#define FA2_H

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. Codes 0-7 are the plain entry point's; FA2_ERR_ALIAS and
 * FA2_ERR_ARG were added after them for the aliasing check and the arguments
 * of the extended entry points, so the first eight keep their values.
 * Argument checks run in this order before any HIP call:
 *   NULLPTR, SHAPE, SCALE, ARG, ALIGN, OVERFLOW, ALIAS,
 * so every code except FA2_ERR_DEVICE and FA2_ERR_LAUNCH is reported without
 * touching a GPU; the device check (DEVICE) and the launch (LAUNCH) follow. */
typedef enum {
    FA2_OK = 0,
    FA2_ERR_NULLPTR = 1,   /* a tensor pointer (or cu_seqlens) is NULL                     */
    FA2_ERR_SHAPE = 2,     /* a size < 1, D not 64 or 128, H not a multiple of H_kv, or
                              causal not 0 or 1                                            */
    FA2_ERR_SCALE = 3,     /* scale is not finite or not > 0                                */
    FA2_ERR_ALIGN = 4,     /* q, k, v or o not 16-byte aligned; lse or cu_seqlens not 4-byte */
    FA2_ERR_OVERFLOW = 5,  /* sequence length >= 2^29, more than 2^31-1 workgroups (counted
                              at the smallest workgroup height, 128 query rows), or a packed
                              K/V row stride (H_kv*D) too large for 32-bit offsets          */
    FA2_ERR_DEVICE = 6,    /* no current HIP device, or it is not a gfx950 GPU            */
    FA2_ERR_LAUNCH = 7,    /* the kernel launch failed (the status hipLaunchKernel returned) */
    FA2_ERR_ALIAS = 8,     /* o or lse overlaps q, k, v (or cu_seqlens), or each other      */
    FA2_ERR_ARG = 9        /* a window side < -1, or dropout_p not in [0, 1)                */
} fa2_status;

/*
 * fa2_fwd -- enqueue one attention forward pass on `stream`.
 *
 *   q, k, v  device pointers to fp16 (IEEE binary16 bits), each a contiguous
 *            [B, H, S, D] tensor: element (b,h,s,d) at ((b*H + h)*S + s)*D + d.
 *   o        device pointer, fp16 output, same layout as q.
 *   lse      device pointer, fp32 output [B, H, S]: element (b,h,s) at
 *            (b*H + h)*S + s; the natural-log log-sum-exp of row s's scaled
 *            scores over its admissible keys.
 *   B, H, S  batch, heads, sequence length (queries and keys alike), each >= 1.
 *   D        head dimension, 64 or 128.
 *   causal   0: every key is admissible; 1: key j is admissible for query i
 *            only when j <= i.
 *   scale    softmax scale applied to q_i . k_j; finite and > 0 (the kernel
 *            takes the row maximum on unscaled scores and scales afterwards,
 *            which is exact only for a positive scale).
 *   stream   a hipStream_t of the current HIP device (the pointers are that
 *            device's memory), or NULL for its default stream. The device
 *            check and the launch use the current device.
 *
 * Ownership: the caller allocates and owns every buffer; the library allocates
 * no device memory and keeps no state besides per-device "is gfx950" and
 * "large LDS enabled" flags. The call is asynchronous: it returns after the
 * launch, and o/lse are valid once `stream` has been synchronised. Inputs are
 * only read. The function is thread-safe. o and lse must not overlap q, k, v
 * or each other (checked).
 *
 * Returns FA2_OK or one of the codes above; on an error nothing is enqueued.
 */
int fa2_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
            int B, int H, int S, int D, int causal, float scale, void *stream);

/*
 * fa2_fwd_ex -- fa2_fwd with GQA/MQA, a local window and dropout.
 *
 *   q, o          fp16 [B, H, S, D] contiguous, as in fa2_fwd.
 *   k, v          fp16 [B, H_kv, S, D] contiguous.
 *   lse           fp32 [B, H, S], as in fa2_fwd.
 *   H_kv          K/V heads, >= 1, dividing H.
 *   window_left, window_right
 *                 the admissible keys of query i are
 *                 max(0, i - window_left) .. min(S-1, i + window_right);
 *                 -1 leaves a side unbounded. fa2_fwd(causal) is (-1, causal ? 0 : -1).
 *                 Every row admits at least its own key, so no row is empty.
 *   dropout_p     probability of dropping an attention weight, 0 <= p < 1;
 *                 0 disables dropout (no random numbers are drawn).
 *   seed, offset  Philox key and fourth counter word (see the top of this file);
 *                 the same arguments give bit-identical outputs.
 *   scale, stream as in fa2_fwd.
 *
 * Ownership, asynchrony and errors as fa2_fwd.
 */
int fa2_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int H, int H_kv, int S, int D,
               int window_left, int window_right,
               float dropout_p, unsigned long long seed, unsigned int offset,
               float scale, void *stream);

/*
 * fa2_fwd_varlen -- attention over sequences of different lengths packed
 * along the row axis.
 *
 *   q, o          fp16 [total, H, D] contiguous: row r of head h at (r*H + h)*D.
 *   k, v          fp16 [total, H_kv, D] contiguous.
 *   lse           fp32 [H, total]: element (h, r) at h*total + r.
 *   cu_seqlens    device int32 [num_seqs + 1]: sequence s occupies rows
 *                 cu_seqlens[s] .. cu_seqlens[s+1]-1. It must start at 0, be
 *                 non-decreasing and end at `total`; sequences may be empty.
 *                 It is read on the device only. Entries are clamped to
 *                 [0, total] and lengths to max_seqlen, so a malformed table
 *                 never makes the kernel address memory outside the tensors,
 *                 but the rows it does not cover are then left unwritten.
 *   num_seqs      number of sequences, >= 1.
 *   total         rows of the packed tensors, >= 1.
 *   max_seqlen    >= the longest sequence (>= 1); it sizes the grid.
 *   H, H_kv, D, window_left, window_right, dropout_p, seed, offset, scale, stream
 *                 as in fa2_fwd_ex; for dropout, b is the sequence index and
 *                 i, j are rows counted from the sequence start.
 *
 * Ownership, asynchrony and errors as fa2_fwd; cu_seqlens must not overlap o
 * or lse (checked).
 */
int fa2_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                   const int *cu_seqlens, int num_seqs, int total, int max_seqlen,
                   int H, int H_kv, int D, int window_left, int window_right,
                   float dropout_p, unsigned long long seed, unsigned int offset,
                   float scale, void *stream);

/* A static, human-readable name for a return code (never NULL). */
const char *fa2_strerror(int status);

/*
 * fa2_kernel_config -- describe the launch fa2_fwd would make, without a GPU.
 * For valid arguments, writes the query rows per workgroup, key rows per
 * LDS ring stage, threads per workgroup, workgroup count and LDS bytes per
 * workgroup, and returns FA2_OK; otherwise returns the same code fa2_fwd would
 * for those sizes (pointer, device and launch checks excepted). Any output
 * pointer may be NULL.
 */
int fa2_kernel_config(int B, int H, int S, int D, int causal, int *rows_per_block,
                      int *keys_per_tile, int *threads_per_block, long long *blocks,
                      int *lds_bytes);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */

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
 * Precision: fp16 inputs, fp32 accumulation (MFMA), fp32 softmax state, fp16
 * output rounded to nearest even, fp32 LSE.
 */
#ifndef FA2_H
#define FA2_H

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. Argument checks run in this order before any HIP call, so
 * every code up to FA2_ERR_ALIAS is reported without touching a GPU. */
typedef enum {
    FA2_OK = 0,
    FA2_ERR_NULLPTR = 1,   /* q, k, v, o or lse is NULL                                 */
    FA2_ERR_SHAPE = 2,     /* B, H or S < 1, or D not 64 or 128, or causal not 0 or 1    */
    FA2_ERR_SCALE = 3,     /* scale is not finite or not > 0                              */
    FA2_ERR_ALIGN = 4,     /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
    FA2_ERR_OVERFLOW = 5,  /* S*D >= 2^31, or the grid would exceed 2^31-1 workgroups    */
    FA2_ERR_ALIAS = 6,     /* o or lse overlaps q, k or v, or o overlaps lse              */
    FA2_ERR_DEVICE = 7,    /* the current HIP device is not a gfx950 GPU                  */
    FA2_ERR_LAUNCH = 8     /* the kernel launch failed (hipGetLastError)                  */
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
 *   stream   a hipStream_t, or NULL for the default stream.
 *
 * Ownership: the caller allocates and owns every buffer; the library allocates
 * no device memory and keeps no state besides a per-device "is gfx950" flag.
 * The call is asynchronous: it returns after the launch, and o/lse are valid
 * once `stream` has been synchronised. Inputs are only read. The function is
 * thread-safe. o and lse must not overlap q, k, v or each other (checked).
 *
 * Returns FA2_OK or one of the codes above; on an error nothing is enqueued.
 */
int fa2_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
            int B, int H, int S, int D, int causal, float scale, void *stream);

/* A static, human-readable name for a return code (never NULL). */
const char *fa2_strerror(int status);

/*
 * fa2_kernel_config -- describe the launch fa2_fwd would make, without a GPU.
 * For valid arguments, writes the query rows per workgroup, key rows per
 * tile, threads per workgroup, workgroup count and LDS bytes per workgroup, and
 * returns FA2_OK; otherwise returns the same code fa2_fwd would (device and
 * launch checks excepted). Any output pointer may be NULL.
 */
int fa2_kernel_config(int B, int H, int S, int D, int causal, int *rows_per_block,
                      int *keys_per_tile, int *threads_per_block, long long *blocks,
                      int *lds_bytes);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */

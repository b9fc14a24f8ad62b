/*
 * fa355.h -- FlashAttention forward pass for AMD Instinct MI355X (gfx950).
 *
 * One call computes exact scaled-dot-product attention
 *
 *     O = softmax(Q K^T * scale) V,      lse = logsumexp of each scaled score row
 *
 * ("FlashAttention (VI)", section "Vấn đề của cơ chế attention tiêu chuẩn", eq.
 * Attention) in a single fused kernel: Q is split into row tiles, K and V stream
 * through on-chip memory in row blocks, and the running row maximum, row sum and
 * rescaled output stay on chip through the online-softmax recurrence ("MCU 上
 * Transformer 模型的 Flash Attention 实现…", §二, flowchart and merge equations;
 * "FlashAttention (VI)", sections on tiling, online softmax and kernel fusion).
 * The N x N score matrix never reaches device memory, and the library allocates
 * nothing: memory use is the caller's O(N) tensors only ("FlashAttention 在昇腾 NPU
 * 上是怎么省显存的？", tiling section: only two rows of softmax statistics are kept).
 *
 * Tensor layout follows the pages' user API, [batch, heads, seq_len, head_dim]
 * ("FlashAttention 在昇腾 NPU 上…", section on running the operator):
 *   q, o : [B, Hq,  N, d]    contiguous, d innermost
 *   k, v : [B, Hkv, N, d]    contiguous, d innermost
 *   lse  : [B, Hq,  N]       fp32, natural log, in units of scaled scores
 * Grouped-query attention is expressed by the K/V head count alone (same page,
 * pitfall 4; "深度探索Flash-Attention中GQA性能调优技术解析", GQA mechanism): query head
 * h reads K/V head h / (Hq / Hkv), i.e. Hq/Hkv consecutive query heads share one.
 * Causal masking lets query row i see key rows j <= i (same Ascend page, pitfall 1).
 *
 * Ownership: the caller allocates and frees every buffer; pointers are device
 * pointers.  Asynchrony: a successful call enqueues exactly one kernel on `stream`
 * (NULL = the null stream) and returns; results are valid once the stream has
 * reached that point.  Calls are reentrant and thread-safe; the library keeps no
 * mutable state apart from fa_fwd_decode_noalloc's per-GPU workspace.  Errors: arguments are validated before any HIP call; on any
 * error the call returns a negative fa355_status and leaves o and lse untouched.
 * Empty calls: with no query rows (B = 0, or N = 0; Nq = 0 for fa_fwd_decode) every
 * entry point returns FA355_OK at once, enqueues nothing and touches no buffer, so
 * any pointer may be NULL; only the sizes are checked (none negative, Hq and Hkv
 * >= 1 with Hq % Hkv == 0).
 * Size limits (FA355_ERR_SHAPE beyond them): every tensor a call touches holds at
 * most 2^40 elements, and one head of each tensor fits the kernels' 32-bit byte
 * offsets (N d elem_bytes <= 2^31 - 1 - 65536; each entry point states its own).
 * Each kernel launch a call makes must also have fewer than 2^32 work-items along
 * each grid dimension (HIP's limit): e.g. the plain forward launches about
 * 2 B Hq N work-items, the decoding merge 256 per (batch, head, query) row.  A
 * call past that is FA355_ERR_SHAPE, found before any HIP call.
 * There is no silent fallback: an unsupported head dimension, dtype or tiling is an
 * error, never a slower path (contrast "FlashAttention…昇腾…" page 2, pitfall).
 */
#ifndef FA355_H
#define FA355_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA355_F32 = 0,
    FA355_F16 = 1,
    FA355_BF16 = 2
} fa355_dtype;

typedef enum {
    FA355_OK = 0,
    FA355_ERR_NULL = -1,        /* q, k, v or o is NULL                                   */
    FA355_ERR_SHAPE = -2,       /* B or N < 0, Hq or Hkv < 1, Hq % Hkv != 0, or too large */
    FA355_ERR_UNSUPPORTED = -3, /* head dim, dtype pair or tiling not built               */
    FA355_ERR_ALIGN = -4,       /* q, k, v, o not 16-byte aligned, or lse not 4-byte      */
    FA355_ERR_ARG = -5,         /* non-finite scale; o or lse overlapping another buffer  */
    FA355_ERR_HIP = -6          /* the HIP launch reported an error                        */
} fa355_status;

/* Tile sizes: br = query rows per workgroup, bc = key/value rows per step.
 * {0, 0} (or a NULL pointer) selects the built-in choice for the shape. */
typedef struct {
    int br;
    int bc;
} fa355_tuning;

/* What a call would launch; filled by fa_fwd_check. */
typedef struct {
    int br;            /* query rows per workgroup                     */
    int bc;            /* key/value rows per step                      */
    int waves;         /* 64-lane wavefronts per workgroup             */
    int grid;          /* workgroups launched                          */
    int lds_bytes;     /* LDS per workgroup                            */
} fa355_plan;

/*
 * Forward attention, output in the input dtype.
 *   q, k, v   device pointers, layouts above, element type `dtype`
 *   o         device pointer [B,Hq,N,d] of `dtype`; written
 *   lse       device pointer [B,Hq,N] fp32, or NULL to skip it
 *   B, Hq, Hkv, N, d   sizes; d in {64, 128, 256} for F16/BF16, d = 64 for F32
 *   causal    nonzero: query i sees keys j <= i
 *   scale     multiplies Q K^T; any finite value (1/sqrt(d) is the usual one)
 *   stream    HIP stream to enqueue on
 * Returns FA355_OK or a negative fa355_status.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           fa355_dtype dtype, hipStream_t stream);

/*
 * As fa_fwd, plus:
 *   o_dtype   the output element type: in_dtype, or FA355_F32 for F16/BF16 inputs
 *             (identical arithmetic; only the final store differs)
 *   tuning    NULL or {0,0} for the default tiles, else one of the built tilings
 *             (br, bc): for F16/BF16 with d = 64 or 128, (128,64), (128,32), (256,64)
 *             (also with F32 output) and (64,64); with d = 256, (128,32) (the
 *             default: a score and an output wavefront per 32 query rows) and
 *             (128,64) (wavefront pairs), each also with F32 output;
 *             for F32, (32,32), (64,32), (128,32)
 */
int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
              fa355_dtype in_dtype, fa355_dtype o_dtype,
              const fa355_tuning *tuning, hipStream_t stream);

/*
 * Validation only: runs every check fa_fwd_ex runs, makes no HIP call and
 * launches nothing.  On FA355_OK and a non-NULL `plan`, fills in the launch the
 * call would make.  Pointers are only compared and tested for alignment, never
 * dereferenced, so host addresses may be passed.
 */
int fa_fwd_check(const void *q, const void *k, const void *v, const void *o,
                 const float *lse, int B, int Hq, int Hkv, int N, int d, int causal,
                 float scale, fa355_dtype in_dtype, fa355_dtype o_dtype,
                 const fa355_tuning *tuning, fa355_plan *plan);

/*
 * Forward with an additive bias on the scaled scores:
 *     O = softmax(Q K^T * scale + bias) V
 * (the fused additive bias / general mask of the FlashAttention feature lists:
 * "深度探索Flash-Attention中GQA性能调优技术解析", and "FlashAttention (VI)" on
 * FlashAttention-3).  A bias of -inf masks a (query, key) pair, so any mask can be
 * given this way; a query row left with no finite score gets O = 0 and lse = -inf.
 * Causal masking, if asked for, applies on top.
 *   bias       device pointer, element type `dtype`; element (b, h, i, j) -- batch,
 *              query head, query row, key -- at b*bias_stride_b + h*bias_stride_h +
 *              i*bias_stride_row + j.  A stride of 0 shares the bias across that
 *              dimension (e.g. one [N,N] bias for every batch and head).
 *   strides    in elements; bias_stride_row >= N; all strides multiples of 4 and
 *              bias 8-byte aligned (FA355_ERR_ALIGN); negative strides or a row
 *              stride below N are FA355_ERR_ARG; a bias whose extent (last element
 *              addressed, plus one) exceeds 2^40 elements is FA355_ERR_SHAPE
 *   dtype      F16 or BF16; d in {64, 128}; output in the input dtype
 * Otherwise as fa_fwd.  Reads the bias once per (query row, key) it needs:
 * B*Hq*N^2*2 bytes (halved when causal) on top of the forward's traffic.
 */
int fa_fwd_bias(const void *q, const void *k, const void *v, void *o, float *lse,
                const void *bias, long long bias_stride_b, long long bias_stride_h,
                long long bias_stride_row, int B, int Hq, int Hkv, int N, int d, int causal,
                float scale, fa355_dtype dtype, hipStream_t stream);

/*
 * Split-KV forward: as fa_fwd (output in the input dtype), with each query tile's
 * key/value range cut into num_splits contiguous pieces handled by separate
 * workgroups, for shapes with too few query tiles to fill the GPU.  Partial
 * results are combined exactly by the online-softmax merge rule ("MCU 上
 * Transformer 模型的 Flash Attention 实现…", §二, merge equations):
 * lse = log sum_s e^{lse_s}, O = sum_s e^{lse_s - lse} O_s.
 *   dtype      F16 or BF16; d in {64, 128}
 *   num_splits 1 .. 16
 *   o_part     device pointer, caller-owned fp32 workspace [num_splits,B,Hq,N,d]
 *   lse_part   device pointer, caller-owned fp32 workspace [num_splits,B,Hq,N]
 * Enqueues two kernels (partials, merge) on `stream`; allocates nothing.  The
 * workspaces must be 16- and 4-byte aligned and overlap nothing else
 * (FA355_ERR_ARG); num_splits out of range is FA355_ERR_ARG.
 */
int fa_fwd_split(const void *q, const void *k, const void *v, void *o, float *lse,
                 int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                 fa355_dtype dtype, int num_splits, float *o_part, float *lse_part,
                 hipStream_t stream);

/*
 * Backward pass: the gradients of sum(O * dout) for O = fa_fwd(q, k, v), i.e. of
 * any loss L with dL/dO = dout ("FlashAttention (VI)", equation Attention,
 * differentiated; the forward pass keeps no N x N matrix for it, as the Ascend
 * page's section on standard attention's memory asks -- P is recomputed from lse).
 *   q, k, v    the forward inputs (layouts above), element type `dtype`
 *   o          the forward output [B,Hq,N,d], element type `dtype`
 *   dout       dL/dO [B,Hq,N,d], element type `dtype`
 *   lse        the forward pass's logsumexp [B,Hq,N] fp32 (natural log, scaled units)
 *   dq         device pointer [B,Hq,N,d] fp32; written with dL/dQ
 *   dk, dv     device pointers [B,Hkv,N,d] fp32; written with dL/dK and dL/dV (for
 *              grouped-query attention, summed over the query heads of each K/V head)
 *   delta      device pointer [B,Hq,N] fp32, a caller-owned workspace; on return it
 *              holds D_i = dout_i . o_i
 *   B .. scale as for fa_fwd (the same scale and causal flag as the forward call);
 *              dtype F16 or BF16, d in {64, 128, 256}
 * All of q, k, v, o, dout, dq, dk, dv must be 16-byte aligned, lse and delta 4-byte
 * aligned; none of dq, dk, dv, delta may overlap each other or any input.
 * Enqueues three kernels on `stream` and returns; allocates nothing (at d = 256 the
 * dK/dV kernel keeps a few registers in the per-lane private memory the HIP runtime
 * provides for every kernel).  Errors as for fa_fwd: validation runs before any HIP
 * call and leaves the outputs untouched.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, float *dq, float *dk, float *dv, float *delta,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           fa355_dtype dtype, hipStream_t stream);

/*
 * Forward with 8-bit floating-point inputs (the FP8 variant of "深度探索Flash-Attention
 * 中GQA性能调优技术解析", FP8 section, and of FlashAttention-3 in "FlashAttention
 * (VI)", section on the evolution of the algorithm): q, k, v hold OCP e4m3 codes (1 sign bit, 4 exponent bits with bias 7, 3
 * fraction bits; largest finite 448; 0x7f and 0xff are NaN), one byte per element,
 * layouts as above.  Each tensor has one fp32 descale: the value of a stored code x
 * is descale * e4m3(x).  Computes the forward pass on those values:
 *     O = softmax((q_descale q)(k_descale k)^T * scale) (v_descale v)
 *   o          device pointer [B,Hq,N,d] bf16; written
 *   lse        device pointer [B,Hq,N] fp32 (natural log, scaled units), or NULL
 *   q_descale, k_descale, v_descale   finite and > 0 (else FA355_ERR_ARG)
 *   d          64 or 128
 * The attention weights are rounded to e4m3 for the P V product (relative error up
 * to 2^-4 per weight, before normalisation by the unrounded row sum); lse is taken
 * from the unrounded weights.  Otherwise as fa_fwd: one kernel, nothing allocated,
 * validation before any HIP call.
 */
int fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int Hq, int Hkv, int N, int d, int causal, float scale,
               float q_descale, float k_descale, float v_descale, hipStream_t stream);

/*
 * Decoding against a key/value cache: Nq new queries per head against Nk cached
 * keys and values, for Nq much smaller than Nk.
 *   q, o       device pointers [B,Hq,Nq,d], element type `dtype`
 *   k, v       device pointers [B,Hkv,Nk,d]
 *   lse        device pointer [B,Hq,Nq] fp32, or NULL
 *   causal     nonzero: the queries are the last Nq of the Nk positions, so query i
 *              sees keys j <= i + Nk - Nq (requires Nq <= Nk, else FA355_ERR_SHAPE);
 *              zero: every query sees every key
 *   dtype      F16 or BF16; d in {64, 128}
 *   num_splits 1 .. 256 pieces of the key range, each handled by its own workgroup
 *   o_part     caller-owned fp32 workspace [num_splits,B,Hq,Nq,d]
 *   lse_part   caller-owned fp32 workspace [num_splits,B,Hq,Nq]
 * The Hq/Hkv query heads that share a K/V head are computed together, their
 * (Hq/Hkv)*Nq (head, query) rows packed into one 32-row tile (the PackGQA scheme of
 * "深度探索Flash-Attention中GQA性能调优技术解析", PackGQA section), so
 * (Hq/Hkv)*Nq <= 32 is required (else FA355_ERR_UNSUPPORTED).  Partial results over
 * the key pieces merge exactly as in fa_fwd_split.  Enqueues two kernels on
 * `stream`; allocates nothing; validation as for fa_fwd_split.
 */
int fa_fwd_decode(const void *q, const void *k, const void *v, void *o, float *lse,
                  int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                  fa355_dtype dtype, int num_splits, float *o_part, float *lse_part,
                  hipStream_t stream);

/*
 * fa_fwd_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The partial results go to a workspace the library holds in a
 * static device array of FA355_NOALLOC_SCRATCH_BYTES per GPU (each GPU the library
 * runs on keeps its copy until the process ends): num_splits*B*Hq*Nq*d fp32 partial
 * outputs, rounded up to 256 bytes, then num_splits*B*Hq*Nq fp32 partial lse values.
 * A call whose workspace would exceed that size returns FA355_ERR_SHAPE before any
 * HIP call.  Arguments, layouts, results and the kernels run are those of
 * fa_fwd_decode; the workspace needs no clearing (every entry the merge reads is
 * written by the same call).  Calls nothing that allocates (no hipMalloc, no hipFree);
 * the workspace used is that of the GPU `stream` runs on, its address looked up on the
 * first call for that GPU (FA355_ERR_HIP if the lookup fails).  All calls on one GPU
 * share its workspace: calls that overlap in time
 * on one GPU (on different streams, or from different threads) race and may return
 * each other's partial results; serialise them, e.g. on one stream.
 */
#define FA355_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_fwd_decode_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                          float scale, fa355_dtype dtype, int num_splits, hipStream_t stream);

/* A static, human-readable name for a status code ("unknown status" otherwise). */
const char *fa_status_str(int status);

/* Library version as 10000*major + 100*minor + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */

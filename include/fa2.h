/*
 * fa2.h -- C ABI of the exact-attention forward pass (FlashAttention-2 style)
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation.  For every batch b, head h and query row i,
 *
 *     O[b,h,i,:] = sum_{j visible to i} softmax_j(scale * Q[b,h,i,:] . K[b,h,j,:]) * V[b,h,j,:]
 *     LSE[b,h,i] = ln sum_{j visible to i} exp(scale * Q[b,h,i,:] . K[b,h,j,:])
 *
 * where every key j is visible when causal == 0 and keys j <= i are visible
 * when causal == 1.  This is standard softmax attention (search-result page on
 * the FlashAttention-2 paper, snippet "0x01 Standard Self-Attention"), computed
 * exactly but in tiles with an online softmax, without ever storing the N x N
 * score matrix ("FlashAttention v2 better parallelism + work partitioning"
 * diagram, concept pseudo-code panel; the same page states the method is exact
 * and needs O(N) extra memory).  LSE is the natural-log log-sum-exp of the
 * scaled, masked scores of each row; the pages do not define it, it is the
 * per-row statistic a backward pass needs.
 *
 * Layouts.  q, k, v and o are contiguous row-major [B, H, N, d] tensors of the
 * selected 16-bit dtype (fp16 or bf16; element (b,h,i,t) at offset
 * ((b*H + h)*N + i)*d + t).  lse is a contiguous [B, H, N] float32 tensor.
 * Query and key lengths are equal (self-attention shapes).  N need not be a
 * multiple of any tile size.
 *
 * Arithmetic.  Both products run on the MFMA units with 16-bit inputs and
 * fp32 accumulation; the softmax runs in fp32.  P is rounded to the input
 * dtype (round-to-nearest-even) before the P.V product; the row sum is taken
 * over the fp32 P.  O is written rounded to nearest even in the input dtype.
 *
 * Ownership and execution.  All tensor pointers are DEVICE pointers owned by
 * the caller.  The library allocates no memory, frees nothing, keeps no
 * pointer after returning and needs no workspace.  A call only enqueues work
 * on `stream` (0 = the default stream) and returns; the caller synchronises.
 * Results are deterministic: equal inputs give bitwise-equal outputs.  The
 * functions are thread-safe.
 *
 * Errors.  Arguments are validated on the host before any HIP call; when a
 * check fails nothing is launched, o and lse are left untouched and a negative
 * status is returned.  Checks run in this order, the first failure wins:
 * dtype / causal / scale / variant (FA2_ERR_ARG), B, H or N below 1
 * (FA2_ERR_SHAPE: an empty problem is the caller's no-op, the library is not
 * called for it), NULL pointers (FA2_ERR_NULL),
 * d (FA2_ERR_UNSUPPORTED), size limits (FA2_ERR_SHAPE), alignment
 * (FA2_ERR_ALIGN), overlap (FA2_ERR_ALIAS).  Faults that happen while the
 * kernel runs surface at the caller's synchronisation, not here.
 */
#ifndef FA2_H
#define FA2_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum fa2_status {
    FA2_OK = 0,
    FA2_ERR_NULL = -1,        /* a tensor pointer is NULL                                  */
    FA2_ERR_SHAPE = -2,       /* B, H or N < 1, or a tensor or one head is too large       */
    FA2_ERR_UNSUPPORTED = -3, /* d is not 64 or 128                                         */
    FA2_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned                    */
    FA2_ERR_ARG = -5,         /* scale not finite, causal not 0/1, bad dtype or variant     */
    FA2_ERR_ALIAS = -6,       /* an output overlaps an input or another output              */
    FA2_ERR_LAUNCH = -7       /* the HIP runtime reported an error when launching           */
};

/* Element type of q, k, v and o. */
enum fa2_dtype {
    FA2_DTYPE_FP16 = 0,
    FA2_DTYPE_BF16 = 1
};

/*
 * fa2_fwd_fp16 / fa2_fwd_bf16 -- the forward pass for one element type.
 *
 *   q, k, v  [in]  device, [B,H,N,d] fp16 (resp. bf16), 16-byte aligned
 *   o        [out] device, [B,H,N,d] same dtype, 16-byte aligned, must not
 *                  overlap any other argument
 *   lse      [out] device, [B,H,N] float32, 16-byte aligned, must not overlap
 *                  q, k, v or o
 *   B, H, N        batch, heads, sequence length; each >= 1.
 *                  N*d*2 bytes (one head) must stay below 2^32 and B*H*N*d
 *                  below 2^62.
 *   d              head dimension: 64 or 128
 *   causal         0: every key visible; 1: key j visible to query i iff j <= i
 *   scale          multiplies q.k before the softmax; any finite value
 *                  (0 gives uniform weights; negative values are allowed)
 *   stream         HIP stream the kernel is enqueued on (0 = default stream)
 *
 * Returns FA2_OK or a negative fa2_status.
 */
int fa2_fwd_fp16(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, int causal, float scale, hipStream_t stream);
int fa2_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/* fa2_fwd -- the same twelve arguments plus dtype (an fa2_dtype value). */
int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            int B, int H, int N, int d, int causal, float scale, hipStream_t stream, int dtype);

/*
 * fa2_fwd_variant -- the forward pass with an explicit tile configuration,
 * for tuning sweeps and tiling-invariance tests.  variant 0 is the tuned
 * default that fa2_fwd uses; 1 .. fa2_num_variants()-1 select the entries
 * described by fa2_variant_name().  Every variant computes the same function;
 * results agree to rounding.  Returns FA2_ERR_ARG for an unknown variant.
 */
int fa2_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, int causal, float scale, hipStream_t stream,
                    int dtype, int variant);

/*
 * fa2_fwd_check -- run exactly the argument validation of fa2_fwd_variant and
 * return its status, without launching anything or calling the HIP runtime.
 */
int fa2_fwd_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  int B, int H, int N, int d, int causal, float scale, int dtype, int variant);

/*
 * fa2_bwd -- the backward pass: gradients of the forward pass's O with
 * respect to q, k and v, given the upstream gradient dO.
 *
 * The pages name the backward pass as the step after the forward one
 * ("FlashAttention v4 Blackwell pipeline co-design" diagram: its list of v4
 * directions and the backward note under its pseudo-code panel, which aim to
 * remove the atomic accumulation of dQ; a snippet of the search-result page
 * for the FlashAttention-2 paper lists backward support) but print no
 * formulas.  The gradients are those of the forward definition above.  With
 * S = scale * Q K^T (masked as in the forward pass), P = exp(S - LSE) (the
 * softmax rows, recomputed from the saved LSE), D_i = sum_t dO[i,t] O[i,t]:
 *
 *     dV = P^T dO      dS = P * (dO V^T - D)      dQ = scale * dS K      dK = scale * dS^T Q
 *
 *   q, k, v  [in]  device, [B,H,N,d] fp16 or bf16 (dtype), 16-byte aligned
 *   o        [in]  device, [B,H,N,d]: the forward pass's output for q, k, v
 *   lse      [in]  device, [B,H,N] float32: the forward pass's LSE
 *   dout     [in]  device, [B,H,N,d]: the upstream gradient dO
 *   dq, dk, dv [out] device, [B,H,N,d] same dtype (rounded to nearest even)
 *   delta    [out] device, [B,H,N] float32: D_i = rowsum(dO * O), in fp32
 *                  (also consumed by the call itself)
 *   B, H, N, d, causal, scale, stream, dtype: as for fa2_fwd; scale and
 *                  causal must be the values the forward pass used.
 *
 * Every pointer is 16-byte aligned and owned by the caller; no output may
 * overlap an input or another output.  The call enqueues three kernels on
 * stream (D, then dK and dV, then dQ; variant 10 of fa2_bwd_variant enqueues
 * two: dQ, which also computes D, then dK and dV) and allocates nothing: dQ is computed
 * by its own kernel over query blocks instead of by atomic adds across key
 * blocks, so results are deterministic.  Validation and error codes as for
 * fa2_fwd (NULL, shape, d, alignment, overlap, argument), before any HIP
 * call; on failure nothing is launched and no output is written.
 */
int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
            const void* dout, void* dq, void* dk, void* dv, float* delta,
            int B, int H, int N, int d, int causal, float scale, hipStream_t stream, int dtype);

/* fa2_bwd_fp16 / fa2_bwd_bf16 -- fa2_bwd for one element type. */
int fa2_bwd_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, float* delta,
                 int B, int H, int N, int d, int causal, float scale, hipStream_t stream);
int fa2_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, float* delta,
                 int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * fa2_bwd_variant -- fa2_bwd with an explicit kernel configuration for the
 * dK/dV step, for tuning and for tests that every configuration computes the
 * same gradients.  variant 0 is the default that fa2_bwd uses; the others are
 * described by fa2_bwd_variant_name():
 *   1 "dkdv_w4_occ1": 4 waves x 32 keys per workgroup, one wave per SIMD,
 *     each wave accumulating both dK and dV of its keys;
 *   2 "dkdv_w8_split_occ2": 8 waves, two per SIMD, the two waves of a SIMD
 *     own the same 32 keys, one accumulating dV and the other dK (both
 *     recompute S = Q K^T);
 *   3 "dkdv_w8_split_occ2_ring4": variant 2 with its query tiles copied
 *     straight from memory into a 4-stage LDS ring, three tiles ahead;
 *   4 "dkdv_w8_split_occ2_ring4_dq_ring3", 5 "dkdv_w4_occ1_dq_ring3":
 *     variants 3 and 1 with the dQ kernel's key tiles copied straight from
 *     memory into a 3-stage LDS ring, two tiles ahead (variants 1-3 stage
 *     them through registers, one tile ahead);
 *   6 "dkdv_w8_split_occ2_ring4_q64": variant 3 with 64-query tiles, each
 *     processed as two 32-query sub-blocks between two barriers;
 *   7 "dkdv_w8_pair_occ2_ring3_q64": the dV wave of a SIMD computes S and P
 *     and hands the fp32 P to the dK wave through LDS, so no product is
 *     computed twice; 64-query tiles on a 3-stage copy ring;
 *   8 "dkdv_w8_pair_occ2_ring3_q64_dq_look4": variant 7 with the dQ
 *     kernel's MFMAs issued in a fixed order, 4 operand reads ahead;
 *   9 "dkdv_w8_pair_occ2_ring3_q64_look4_dq_look4": variant 8 with the
 *     dK/dV kernel's MFMAs ordered the same way;
 *   10 "dkdv_w8_pair_occ2_ring3_q64_look4_dq_look4_fused_d": variant 9 with
 *     D computed inside the dQ kernel, which then runs first (two kernels
 *     instead of three; delta is written all the same);
 *   11 "dkdv_w4_occ1_dq_w4_look4": variant 1 with 4-wave (128-query) dQ
 *     workgroups at d = 64 (twice the workgroups for small grids); at
 *     d = 128 it is variant 1;
 *   12, 13: variant 9 with 2 and 6 operand reads ahead instead of 4;
 *   14 "dkdv_w8_pipe_occ2_ring3_q64_look2_dq_look4": the P hand-off
 *     pipelined across query tiles, one barrier per iteration (P passed as
 *     16-bit values, dK/dV MFMAs two operand reads ahead).
 *   15 "dkdv_w8_pipe_occ2_ring3_q64_look2_dq_pipe_look4": variant 14 with
 *     the dQ kernel pipelined across key tiles too (dQ of tile j-1 from
 *     dS kept in registers, then S, dP, dS of tile j; 4-stage K/V ring).
 * The default is variant 14 for d = 128, variant 1 for non-causal d = 64 and
 * variant 11 for causal d = 64.
 * Returns FA2_ERR_ARG for an unknown variant.
 */
int fa2_bwd_variant(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, float* delta,
                    int B, int H, int N, int d, int causal, float scale, hipStream_t stream,
                    int dtype, int variant);

/* Number of backward variants (including the default, 0). */
int fa2_bwd_num_variants(void);

/* Static name of a backward variant ("default" for 0), or NULL when out of range. */
const char* fa2_bwd_variant_name(int variant);

/*
 * fa2_bwd_check -- run exactly the argument validation of fa2_bwd and return
 * its status, without launching anything or calling the HIP runtime.
 */
int fa2_bwd_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, const void* dq, const void* dk, const void* dv,
                  const float* delta, int B, int H, int N, int d, int causal, float scale,
                  int dtype);

/*
 * fa2_default_variant -- the variant index (>= 1) that variant 0 resolves to
 * for this dtype, d and causal flag, or FA2_ERR_ARG / FA2_ERR_UNSUPPORTED.
 */
int fa2_default_variant(int dtype, int d, int causal);

/* Number of tile variants (including the default, 0). */
int fa2_num_variants(void);

/* Static description of a variant ("default" for 0), or NULL when out of range. */
const char* fa2_variant_name(int variant);

/* Static text for a status code; never NULL. */
const char* fa2_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fa2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */

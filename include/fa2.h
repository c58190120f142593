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
 * fa2_fwd_fp8 -- the forward pass with FP8 inputs.
 *
 * The pages name FP8 arithmetic as a hardware capability that v2 leaves
 * unused ("FlashAttention v2 better parallelism + work partitioning"
 * diagram, panel on what v2 changes) but give no FP8 scheme; this one is:
 *
 *   q, k, v  [in]  device, [B,H,N,d] 8-bit codes in the OCP E4M3 format
 *                  (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *                  largest finite magnitude 448; S.1111.111 is NaN),
 *                  16-byte aligned.  The inputs are decode(q) * descale_q,
 *                  decode(k) * descale_k and decode(v) * descale_v.
 *   o        [out] device, [B,H,N,d] bf16 (round to nearest even), 16-byte
 *                  aligned, must not overlap any other argument
 *   lse      [out] device, [B,H,N] float32, 16-byte aligned, must not
 *                  overlap q, k, v or o
 *   B, H, N, d, causal, scale, stream: as for fa2_fwd_fp16; N*d*2 bytes
 *                  (one head of o) must stay below 2^32
 *   descale_q, descale_k, descale_v: finite float32 factors, one per tensor
 *
 * O and LSE are those of the definition at the top of this file applied to
 * the dequantised inputs, except for one rounding step: the probabilities
 * enter the P.V product as E4M3 values.  Per tile of 8192/d keys (64 keys at
 * d = 128, 128 at d = 64, in key order) and per row, P = 2^(6 + c*s - m)
 * with c = scale * descale_q * descale_k * log2(e) and m the row's
 * reference max, which moves to the tile's max only when that exceeds it
 * by more than 2.75, is rounded to the nearest E4M3 value (ties to even);
 * the row sum l takes the unrounded P.  Both products accumulate in fp32.
 * Errors: as for fa2_fwd; scale, any descale, or c not finite in float32
 * is FA2_ERR_ARG.
 */
int fa2_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int N, int d, int causal, float scale,
                float descale_q, float descale_k, float descale_v, hipStream_t stream);

/*
 * fa2_fwd_fp8_check -- run exactly the argument validation of fa2_fwd_fp8 and
 * return its status, without launching anything or calling the HIP runtime.
 */
int fa2_fwd_fp8_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      int B, int H, int N, int d, int causal, float scale,
                      float descale_q, float descale_k, float descale_v);

/*
 * fa2_fwd_fp8_variant -- fa2_fwd_fp8 with an explicit kernel, for tuning and
 * for tests that compare the kernels.  variant 0 is the default that
 * fa2_fwd_fp8 uses (fa2_fp8_default_variant says which); the others are
 * described by fa2_fp8_variant_name():
 *   1 "tile_by_tile": score, softmax and P.V of one tile between two
 *     barriers, the copy of a later tile in flight;
 *   2 "sched_ring4": d = 128 only (FA2_ERR_UNSUPPORTED otherwise): the
 *     hand-scheduled loop, 8 waves of 32 rows, the softmax of tile j between
 *     the P.V MFMAs of tile j-1 and the score MFMAs of tile j+1.
 * The default is variant 2 for causal d = 128 and variant 1 otherwise.
 * Every variant computes the same function, including where the reference
 * moves; results agree to fp32 summation order.  Returns FA2_ERR_ARG for an
 * unknown variant, otherwise as fa2_fwd_fp8.
 */
int fa2_fwd_fp8_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int N, int d, int causal, float scale,
                        float descale_q, float descale_k, float descale_v, hipStream_t stream,
                        int variant);

/* The argument validation of fa2_fwd_fp8_variant, without launching anything. */
int fa2_fwd_fp8_variant_check(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, int B, int H, int N, int d, int causal, float scale,
                              float descale_q, float descale_k, float descale_v, int variant);

/* Number of FP8 variants (including the default, 0). */
int fa2_fp8_num_variants(void);

/* Static name of an FP8 variant ("default" for 0), or NULL when out of range. */
const char* fa2_fp8_variant_name(int variant);

/* The FP8 variant (>= 1) that variant 0 resolves to for head dimension d and
 * causal (0/1); only d = 64 and 128 are meaningful. */
int fa2_fp8_default_variant(int d, int causal);

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
 * stream (D, then dK and dV, then dQ) and allocates nothing: dQ is computed
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
 * fa2_bwd_variant -- fa2_bwd with an explicit kernel configuration, for
 * tuning and for tests that every configuration computes the same
 * gradients.  variant 0 is the default that fa2_bwd uses; the others are
 * described by fa2_bwd_variant_name():
 *   1 "dkdv_w4_occ1": dK/dV workgroups of 4 waves x 32 keys, one wave per
 *     SIMD, each wave accumulating both dK and dV of its keys; dQ
 *     workgroups of 8 waves x 32 queries;
 *   2 "dkdv_w8_pair_occ2_ring3_q64_look4_dq_look4": dK/dV workgroups of 8
 *     waves, two per SIMD owning the same 32 keys: the dV wave computes S
 *     and P and hands P to the dK wave through LDS, so no product is
 *     computed twice; 64-query tiles on a 3-stage copy ring; the MFMAs of
 *     both kernels issued 4 operand reads ahead;
 *   3 "dkdv_w4_occ1_dq_w4_look4": variant 1 with 4-wave (128-query) dQ
 *     workgroups at d = 64, 4 operand reads ahead (twice the workgroups for
 *     small grids); at d = 128 it is variant 1;
 *   4 "dkdv_w8_pipe_occ2_ring3_q64_look2_dq_look4": the P hand-off of
 *     variant 2 pipelined across query tiles, one barrier per iteration,
 *     dK/dV MFMAs 2 operand reads ahead.
 * The default is variant 4.
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

/*
 * moe_mi355x.h -- C ABI of libmoe_mi355x.so: the MoE expert feed-forward as
 * one grouped operation on an AMD Instinct MI355X (gfx950), in BF16 and
 * MXFP8, forward and backward.
 *
 * Source pages (short tags used below):
 *   [BioNeMo]   "NVIDIA发布BioNeMo MoE配方：八卡B200训练Mixtral-8x7B吞吐提升至
 *               Hugging Face基线 2.21 倍" (scopeai.cc), sections
 *               "MoE训练的瓶颈与TE的对应能力" (bottlenecks), "GroupedLinear",
 *               "MXFP8与融合MLP" (MXFP8 and the fused MLP).
 *   [AutoModel] "英伟达开源MoE加速神器：一行代码，微调快3.7倍"
 *               (openai-hub.com), sections "MoE 微调的痛点" (sparse
 *               activation) and "专家并行" (expert parallelism).
 *
 * Conventions shared by every call
 * --------------------------------
 * Types.  bf16 tensors are passed as uint16_t* (bfloat16 bit patterns);
 * MXFP8 tensors are two uint8_t arrays: E4M3 codes and E8M0 scale bytes (one
 * per 32 consecutive values along the stated axis).  All tensors are dense
 * row-major unless stated otherwise.  Every pointer is a DEVICE pointer on the
 * current HIP device, except the per-expert pointer tables of the grouped
 * MLP calls, which are HOST arrays of device pointers.
 *
 * Ownership.  The caller owns every buffer, including the workspace, whose
 * size moe_workspace_bytes() returns.  The library allocates no device or
 * host memory in these calls and keeps no pointer after it returns; host
 * pointer tables are copied into kernel arguments, so they may be freed on
 * return.  Device buffers must stay valid until the stream has executed the
 * work (ordinary stream semantics).
 *
 * Asynchrony.  Every call only enqueues kernels on `stream` (a hipStream_t;
 * NULL = the default stream) and returns; none synchronizes the host.  The
 * per-expert row counts (split sizes) stay on the device; buffers are sized
 * from the total row count T*k on the host.
 *
 * Errors.  Every call returns a moe_status; it never aborts or throws.  All
 * argument checks happen before any launch, so a call that returns an error
 * has enqueued nothing.  Device-data preconditions (split sizes summing to
 * the row count, expert ids below E, valid permutations) are the caller's
 * duty and are not checked by these calls (moe_check_routing checks them
 * on request).  Data that break them give unspecified results, but the
 * kernels keep every access inside the buffers: split sizes are clamped (a
 * negative size counts as 0, and sizes whose running total passes the row
 * count are cut at it); dest_row entries outside [0, T*k) are skipped; an
 * expert id outside [0, E) receives no gradient.  The one exception is
 * src_token of the gathered calls, whose source row count they are not
 * given: it is read as given.  MOE_ERR_HIP reports a failed launch; the HIP
 * error itself is left for the caller's next hipGetLastError().
 *
 * Alignment.  Tensor base pointers must be 16-byte aligned (MOE_ERR_ALIGN).
 *
 * Threading.  Stateless apart from a cached device-architecture check; calls
 * may be made from several host threads on different streams, provided that
 * they do not share output or workspace buffers.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,         /* a required pointer is NULL                       */
    MOE_ERR_SHAPE = 2,        /* a size is out of range or not a needed multiple */
    MOE_ERR_ALIGN = 3,        /* a tensor pointer is not 16-byte aligned          */
    MOE_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required       */
    MOE_ERR_UNSUPPORTED = 5,  /* current device is not gfx950, or unknown option  */
    MOE_ERR_HIP = 6,          /* a HIP launch or query failed                     */
    MOE_ERR_ARG = 7           /* an enum or flag argument has an invalid value    */
} moe_status;

typedef enum moe_precision {
    MOE_BF16 = 0,             /* BF16 operands, fp32 accumulation                 */
    MOE_MXFP8 = 1,            /* E4M3 operands, E8M0 scale per 32 K-values        */
    MOE_FP8 = 2               /* E4M3 operands, one power-of-two scale per tensor */
} moe_precision;

/* moe_route flags */
#define MOE_ROUTE_RENORM 0u       /* softmax over the k picked logits (default) */
#define MOE_ROUTE_SOFTMAX_ALL 1u  /* softmax over all E logits, taken at the picks */

/* moe_workspace_bytes ops */
typedef enum moe_op {
    MOE_OP_ROUTE = 0,
    MOE_OP_MLP_FWD = 1,
    MOE_OP_MLP_BWD = 2,
    MOE_OP_ROUTER_FWD = 3,    /* T, E, k used */
    MOE_OP_ROUTER_BWD = 4,    /* T, H, E used (k must still be valid) */
    MOE_OP_LINEAR_FWD = 5,    /* grouped_linear_fwd: T = rows, H = in_features K,
                                 I = out_features N, E, precision (k must be 1) */
    MOE_OP_LINEAR_BWD = 6     /* grouped_linear_bwd: as MOE_OP_LINEAR_FWD */
} moe_op;

/* Limits of this version. */
#define MOE_MAX_EXPERTS 64

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int status);

/* 1 if the current HIP device is a gfx950 (MI355X / MI350 class), else 0. */
int moe_device_supported(void);

/*
 * moe_route -- top-k routing, split sizes and the stable permutation.
 * [AutoModel, "MoE 微调的痛点": each token activates only a few experts;
 *  BioNeMo, "GroupedLinear": the grouped call takes per-expert token counts,
 *  split_sizes.]
 *
 * logits       fp32 [T, E]  router logits.
 * T            tokens, 0 <= T, T*k <= INT32_MAX.   E: experts, 1..64.
 * k            picks per token, 1 <= k <= E.
 * flags        MOE_ROUTE_RENORM or MOE_ROUTE_SOFTMAX_ALL.
 * topk_expert  int32 [T, k] out: picked experts, largest logit first; equal
 *              logits go to the lower expert index.  Selection uses the fp32
 *              logits themselves.
 * topk_prob    fp32 [T, k]  out: routing probability of each pick.
 * split_sizes  int32 [E]    out: rows routed to each expert (sum = T*k).
 * expert_offsets int32 [E+1] out: exclusive prefix sum of split_sizes.
 * dest_row     int32 [T, k] out: row of pick (t, j) in the expert-grouped
 *              order; inside an expert, rows follow ascending token index.
 * src_token    int32 [T*k]  out: token of each grouped row.
 * workspace    device scratch of moe_workspace_bytes(MOE_OP_ROUTE, ...) bytes.
 * T = 0 is valid: split_sizes and expert_offsets are written as zeros.
 */
int moe_route(const float* logits, int64_t T, int E, int k, uint32_t flags,
              int32_t* topk_expert, float* topk_prob, int32_t* split_sizes,
              int32_t* expert_offsets, int32_t* dest_row, int32_t* src_token,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_route_noalloc -- moe_route without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * that must not call hipMalloc, harnesses that forbid it).  Same arguments
 * (less the workspace) and the same outputs, bit for bit.  Its scratch (the
 * per-256-token-block expert counts and bases and the picks' ranks, 4 bytes
 * each) lives in a static device array of MOE_ROUTE_NOALLOC_MAX_BYTES that
 * every GPU the library runs on holds until the process ends; the call
 * allocates nothing.  Sizes whose scratch exceeds that, i.e.
 * 4*(T*k + 2*E*ceil(T/256)) rounded up to 256 bytes, return
 * MOE_ERR_WORKSPACE before any launch (T*k up to about two million picks
 * at E = 64).  Every call on one device shares the one array and leaves its
 * contents behind (nothing in it needs clearing between calls): calls that
 * overlap in time on one device, from several streams or host threads, race
 * and must be serialized by the caller.
 */
#define MOE_ROUTE_NOALLOC_MAX_BYTES (8u << 20)
int moe_route_noalloc(const float* logits, int64_t T, int E, int k, uint32_t flags,
                      int32_t* topk_expert, float* topk_prob, int32_t* split_sizes,
                      int32_t* expert_offsets, int32_t* dest_row, int32_t* src_token,
                      hipStream_t stream);

/*
 * moe_route_bwd -- gradient of the router logits from the gradient of the
 * grouped-row probabilities (backward of the probabilities moe_route made).
 * [BioNeMo, "MXFP8与融合MLP": the fused MLP's backward has a matching fused
 *  operation, and ScaledSwiGLU takes the routing probabilities as its scales,
 *  so they receive a gradient; AutoModel, "MoE 微调的痛点": the probabilities
 *  come from the routing of each token to a few experts.]
 * The probability gradient arrives per grouped row (dprob_perm, as
 * grouped_mlp_bwd writes it) together with dest_row, instead of as a [T, k]
 * table: the gather dprob[t][j] = dprob_perm[dest_row[t][j]] is done inside
 * the kernel, so no permuted copy is materialized.
 *
 * topk_prob    fp32 [T, k]  probabilities from moe_route.
 * dprob_perm   fp32 [T*k]   gradient per grouped row (from grouped_mlp_bwd).
 * dest_row     int32 [T, k] from moe_route.
 * topk_expert  int32 [T, k] from moe_route.
 * logits       fp32 [T, E]  required with MOE_ROUTE_SOFTMAX_ALL, else may be NULL.
 * dlogits      fp32 [T, E]  out.  Renormalized softmax: for pick j of token t,
 *              p_j (dp_j - sum_i p_i dp_i); 0 for experts not picked.
 *              Full softmax P: P_e (g_e - sum_j p_j dp_j), g = dp at the picks.
 */
int moe_route_bwd(const float* topk_prob, const float* dprob_perm, const int32_t* dest_row,
                  const int32_t* topk_expert, const float* logits, int64_t T, int E, int k,
                  uint32_t flags, float* dlogits, hipStream_t stream);

/*
 * moe_check_routing -- device check of routing data that the grouped calls
 * take on trust (the optional check of the device-data preconditions above).
 * [AutoModel, "MoE 微调的痛点": each token goes to a few experts; BioNeMo,
 *  "GroupedLinear": the grouped call takes the per-expert row counts.]
 *
 * Checks, on the device and without a host copy of the data:
 *   split_sizes  int32 [E]: every size >= 0 (MOE_CHECK_SPLIT_NEGATIVE) and
 *                their sum == rows (MOE_CHECK_SPLIT_SUM);
 *   dest_row     int32 [T, k]: every entry in [0, rows) (MOE_CHECK_DEST_RANGE);
 *   src_token    int32 [rows]: every entry in [0, T) (MOE_CHECK_SRC_RANGE), and
 *                src_token[dest_row[t][j]] == t (MOE_CHECK_MISMATCH);
 *   topk_expert  int32 [T, k]: every entry in [0, E) (MOE_CHECK_EXPERT_RANGE),
 *                and with split_sizes, dest_row[t][j] inside the rows of expert
 *                topk_expert[t][j] (MOE_CHECK_MISMATCH).
 * Any of the four arrays may be NULL: its checks are skipped.  What moe_route
 * writes passes every check.
 * status       int32 device, out: 0, or the OR of the MOE_CHECK_* bits of the
 *              violations found.  Written by the stream (read it after
 *              synchronizing); the call itself does not synchronize.
 * Errors: MOE_ERR_NULL (status NULL), MOE_ERR_SHAPE (T < 0, rows < 0,
 * E outside 1..64, k outside 1..E with dest_row or topk_expert given).
 */
#define MOE_CHECK_SPLIT_NEGATIVE 1
#define MOE_CHECK_SPLIT_SUM 2
#define MOE_CHECK_DEST_RANGE 4
#define MOE_CHECK_SRC_RANGE 8
#define MOE_CHECK_MISMATCH 16
#define MOE_CHECK_EXPERT_RANGE 32
int moe_check_routing(const int32_t* split_sizes, int E, int64_t rows, const int32_t* dest_row,
                      const int32_t* src_token, const int32_t* topk_expert, int64_t T, int k,
                      int32_t* status, hipStream_t stream);

/*
 * moe_router_fwd -- the router linear layer fused with the routing: logits =
 * x W_r^T, then exactly what moe_route does with those logits.
 * [AutoModel, "MoE 微调的痛点": every token is routed to a few experts.  The
 *  pages do not give the router; it is read as a bias-free linear map of the
 *  token's hidden state, as in the MoE models that page names.]
 *
 * x            bf16 [T, H], H a multiple of 64.   w_router: bf16 [E, H].
 * logits       fp32 [T, E] out: sum_h x[t,h] w_router[e,h] with fp32
 *              accumulation (the order of the sum is unspecified); kept for
 *              moe_route_bwd with MOE_ROUTE_SOFTMAX_ALL and for the caller.
 * k, flags, topk_expert .. src_token, workspace: as moe_route (workspace of
 *              moe_workspace_bytes(MOE_OP_ROUTER_FWD, T, 0, 0, E, k, 0) bytes).
 */
int moe_router_fwd(const uint16_t* x, const uint16_t* w_router, int64_t T, int H, int E, int k,
                   uint32_t flags, float* logits, int32_t* topk_expert, float* topk_prob,
                   int32_t* split_sizes, int32_t* expert_offsets, int32_t* dest_row,
                   int32_t* src_token, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * moe_router_bwd -- backward of the router linear layer, fused with the
 * combine of the expert path's token gradient.
 *
 * dlogits      fp32 [T, E] (moe_route_bwd).   x, w_router: as in the forward.
 * dxp          bf16 [T*k, H] gradient of the grouped rows from grouped_mlp_bwd,
 *              or NULL (then dx holds the router term alone).
 * dest_row     int32 [T, k] (moe_route); required when dxp is given.
 * dx           bf16 [T, H] out: bf16( sum_j dxp[dest_row[t][j]]  (slot order)
 *              + sum_e dlogits[t,e] w_router[e] ), one fp32 sum, one rounding.
 * dw_router    bf16 [E, H] out: sum_t dlogits[t,e] x[t], fp32 partial sums
 *              over fixed token splits added in a fixed order (deterministic);
 *              zeros when T = 0.
 * workspace    moe_workspace_bytes(MOE_OP_ROUTER_BWD, T, H, 0, E, k, 0) bytes.
 */
int moe_router_bwd(const float* dlogits, const uint16_t* x, const uint16_t* w_router, int64_t T,
                   int H, int E, int k, const int32_t* dest_row, const uint16_t* dxp,
                   uint16_t* dx, uint16_t* dw_router, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * moe_permute -- dispatch: copy each token row to the grouped row of every
 * pick, and move the probabilities along.
 * [AutoModel, "专家并行": tokens are sent to the experts that compute them.]
 *
 * x            bf16 [T, H].   H: multiple of 8.
 * dest_row     int32 [T, k]   from moe_route.
 * topk_prob    fp32 [T, k]    may be NULL (then prob_perm is not written).
 * xp           bf16 [T*k, H]  out: xp[dest_row[t][j]] = x[t].
 * prob_perm    fp32 [T*k]     out (may be NULL): prob_perm[dest_row[t][j]] = topk_prob[t][j].
 * x and xp may both be NULL: then only prob_perm is written (topk_prob and
 * prob_perm required), for a consumer that gathers the token rows itself
 * (grouped_mlp_fwd_gather / grouped_mlp_bwd_gather).
 */
int moe_permute(const uint16_t* x, int64_t T, int H, int k, const int32_t* dest_row,
                const float* topk_prob, uint16_t* xp, float* prob_perm, hipStream_t stream);

/*
 * moe_unpermute -- combine: y[t] = sum over j = 0..k-1 (in slot order, fp32)
 * of w_tj * yp[dest_row[t][j]], rounded once to bf16.
 * [AutoModel, "专家并行": results are sent back to their tokens.]
 *
 * topk_prob    fp32 [T, k] weights w_tj, or NULL for w = 1.  The grouped MLP
 *              already applies the routing probability (ScaledSwiGLU), so the
 *              layer passes NULL here; a non-NULL table serves a combine for
 *              experts that did not apply it.
 * yp           bf16 [T*k, H];  y: bf16 [T, H] out.  H: multiple of 8.
 */
int moe_unpermute(const uint16_t* yp, int64_t T, int H, int k, const int32_t* dest_row,
                  const float* topk_prob, uint16_t* y, hipStream_t stream);

/*
 * mxfp8_quantize -- MXFP8 block quantization of a bf16 matrix.
 * [BioNeMo, "MXFP8与融合MLP" and the bottleneck section: 8-bit values with one
 *  scale per 32 consecutive values, made from BF16 before a low-precision GEMM.]
 *
 * Block scale: S = log2(X) + 127 for the smallest power of two X with
 * amax <= 448 X, clamped to [0, 254]; S = 0 for an all-zero block.  Codes:
 * E4M3 (bias 7, max 448, no infinities) of v / X, round to nearest even,
 * sign kept (-0 -> 0x80).  NaN/Inf inputs are outside the contract.
 *
 * x        bf16 [rows, cols].
 * axis=1   rowwise: blocks along the last dim; cols multiple of 32.
 *          codes [rows, cols], scales [rows, cols/32].
 * axis=0   grouped columnwise: the rows form ngroups consecutive groups of
 *          group_sizes[g] rows (device int32 [ngroups]; NULL = one group of
 *          all rows).  Inside a group, blocks of 32 consecutive rows start at
 *          the group's first row; the last block is zero-padded.  Group g is
 *          stored transposed as codes [cols, P_g], P_g = 32*ceil(n_g/32), at
 *          byte offset cols*(P_0+..+P_{g-1}); its scales [cols, P_g/32] at
 *          cols*(P_0+..+P_{g-1})/32.  cols multiple of 8.  The buffers must
 *          hold mxfp8_colwise_bytes(); bytes past the used extent are not
 *          written.
 */
int mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t cols, int axis,
                   const int32_t* group_sizes, int ngroups, uint8_t* codes, uint8_t* scales,
                   hipStream_t stream);

/*
 * mxfp8_quantize_both -- both orientations of mxfp8_quantize from one read of
 * x: the rowwise codes and scales of axis=1 and the grouped columnwise codes
 * and scales of axis=0, byte for byte the same as the two separate calls.
 * [BioNeMo, "MXFP8与融合MLP": a tensor that enters GEMMs contracting along
 *  either axis needs both copies.]
 * cols: multiple of 32.  Buffers, groups and errors as for mxfp8_quantize.
 */
int mxfp8_quantize_both(const uint16_t* x, int64_t rows, int64_t cols,
                        const int32_t* group_sizes, int ngroups, uint8_t* row_codes,
                        uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales,
                        hipStream_t stream);

/*
 * mxfp8_dequantize -- inverse of mxfp8_quantize: out bf16 [rows, cols] =
 * RNE_bf16(decode(code) * 2^(S-127)), the exact value of each code times its
 * block's scale, rounded once to bf16.
 * [BioNeMo, bottleneck section: the naive path turns the 8-bit values back
 *  into a wider format in a separate step after the low-precision GEMM; the
 *  fused MLP avoids it, and this call serves callers that need it.]
 * Layouts, groups (axis 0) and errors as for mxfp8_quantize.
 */
int mxfp8_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     int axis, const int32_t* group_sizes, int ngroups, uint16_t* out,
                     hipStream_t stream);

/* Capacity of the grouped columnwise layout: cols*(rows + 31*ngroups) code
 * bytes and a 32nd of that in scale bytes (host-side, no launch). */
void mxfp8_colwise_bytes(int64_t rows, int64_t cols, int ngroups, size_t* code_bytes,
                         size_t* scale_bytes);

/*
 * Tensors the forward saves for the backward.  Caller-owned device buffers;
 * moe_saved_bytes() gives the size of each member.
 *   a1          bf16 [rows, 2I]: gate_up output before the activation (both modes).
 *   a2          BF16 mode: bf16 [rows, I], the ScaledSwiGLU output.
 *   a2_col_*    MXFP8 (FP8) mode: grouped columnwise MXFP8 of the ScaledSwiGLU
 *               output (groups = experts).
 *   xp_col_*    MXFP8 (FP8) mode: grouped columnwise MXFP8 of xp.
 *
 * 8-bit GEMM operand layout ("row-pair layout").  The 8-bit operands that the
 * library keeps for its GEMMs store an R x K byte matrix (K the contraction
 * axis) so that rows 2p and 2p+1 share 128-byte lines, one line per 64
 * K-bytes: byte (r, k) sits at
 *     (r / 2) * PS(K) + (k / 64) * 128 + (r % 2) * 64 + (k % 64),
 *     PS(K) = 128 * ceil(K / 64),
 * so that one K step of two neighbouring rows is one whole cache line.  The
 * *_col_codes hold, per expert e (group g), the transposed group [cols, n_g]
 * in this layout with K = Q_g = 64*ceil(n_g/64) (padding codes unspecified),
 * at byte offset cols*(Q_0+..+Q_{g-1}).  Their scales are those of
 * mxfp8_quantize axis=0 stored block-major per group ([P_g/32][cols] at
 * offset cols*(P_0+..+P_{g-1})/32, P_g = 32*ceil(n_g/32)), the order the
 * backward GEMMs read.
 *
 * Optional, MXFP8 (FP8) mode (all four or none; otherwise MOE_ERR_ARG): the
 * columnwise MXFP8 of the weights, which the backward's data-gradient GEMMs
 * contract along the other axis than the forward's.
 *   w_gate_up_col_*  expert e's W1 quantized along 2I: codes [H, 2I] in the
 *                    row-pair layout at e*2I*H, scales block-major [2I/32][H]
 *                    (E*2I*H/32 bytes, expert e at e*2I*H/32).
 *   w_down_col_*     W2_e quantized along H: codes [I, H] (row-pair layout) at
 *                    e*H*I, scales [H/32][I] at e*H*I/32.
 * When given, grouped_mlp_fwd writes them in the same pass that quantizes the
 * weights rowwise (each weight is read once), and grouped_mlp_bwd uses them
 * instead of quantizing w_gate_up and w_down again; the weights must then be
 * the same in both calls.  When NULL, the backward quantizes the weights.
 * Members that the mode does not use may be NULL.
 */
typedef struct moe_saved {
    uint16_t* a1;
    uint16_t* a2;
    uint8_t* a2_col_codes;
    uint8_t* a2_col_scales;
    uint8_t* xp_col_codes;
    uint8_t* xp_col_scales;
    uint8_t* w_gate_up_col_codes;
    uint8_t* w_gate_up_col_scales;
    uint8_t* w_down_col_codes;
    uint8_t* w_down_col_scales;
} moe_saved;

/* Bytes of member `member` of moe_saved (0 = a1, 1 = a2, ..., 9 =
 * w_down_col_scales, in declaration order) for grouped_mlp_fwd/bwd with these
 * sizes and precision; 0 for a member the precision does not use or invalid
 * arguments.  Host-side, no launch. */
size_t moe_saved_bytes(int precision, int member, int64_t rows, int H, int I, int E);

/*
 * grouped_mlp_fwd -- all experts' gate_up -> ScaledSwiGLU -> down in one call.
 * [BioNeMo, "GroupedLinear": one grouped GEMM over all local experts, each
 *  with its own weight, gate_up out_features = 2*intermediate, no bias, rows
 *  given with split_sizes; "MXFP8与融合MLP": gate_up, ScaledSwiGLU (SwiGLU
 *  times the routing probability), down, fused with quantization so that no
 *  intermediate is dequantized to memory.]
 *
 * Per expert e with its M_e = split_sizes[e] consecutive rows of xp:
 *   A1 = xp_e W1_e^T (fp32 accumulation); g = A1[:, :I], u = A1[:, I:]
 *   A2 = prob * silu(g) * u;  yp_e = A2 W2_e^T (rounded to bf16).
 * MXFP8 mode quantizes xp and W1 along H, A2 and W2 along I (rowwise; A2 in
 * the gate_up GEMM's epilogue), and also saves the columnwise MXFP8 of xp and
 * A2 for the weight gradients (and of W1 and W2 for the data gradients, when
 * moe_saved holds their buffers).
 * FP8 mode [BioNeMo, bottleneck section: FP8 differs from MXFP8 in the
 * scaling granularity] casts the same operands with one scale per tensor:
 * xp, each W1_e and W2_e, and A2, each from the tensor's own amax (current
 * scaling; the scale rule of an MXFP8 block applied to the whole tensor).
 * A2 is written in bf16 by the gate_up epilogue and cast once its amax is
 * known.  The saved buffers and their layouts are those of MXFP8 mode (every
 * block scale of a tensor holds the tensor's scale); the backward must be
 * called with the same precision.
 *
 * precision    MOE_BF16, MOE_MXFP8 or MOE_FP8.
 * E            experts, 1..64.   H, I: hidden and intermediate sizes,
 *              multiples of 128.
 * rows         T*k, 0 <= rows <= INT32_MAX, with 2I * H * 2 (one expert's
 *              bf16 weight) and max(H, 2I)/32 * 32*(ceil(rows/32) + E) (the
 *              block-major scales of the widest 8-bit activation operand)
 *              below 2^31: rows up to about 2.4 million at the Mixtral shape
 *              (the kernels take every other offset from per-tile or per-step
 *              bases); otherwise MOE_ERR_SHAPE.
 * xp           bf16 [rows, H], expert-grouped (moe_permute).
 * split_sizes  int32 [E] device, sum = rows.
 * w_gate_up    HOST array of E device pointers, each bf16 [2I, H] (rows
 *              [0, I) gate, [I, 2I) up).
 * w_down       HOST array of E device pointers, each bf16 [H, I].
 * prob_perm    fp32 [rows] (moe_permute).
 * yp           bf16 [rows, H] out.
 * saved        caller-owned saved tensors (see moe_saved), written.
 * workspace    moe_workspace_bytes(MOE_OP_MLP_FWD, ...) bytes.
 */
int grouped_mlp_fwd(int precision, int E, int H, int I, int64_t rows, const uint16_t* xp,
                    const int32_t* split_sizes, const uint16_t* const* w_gate_up,
                    const uint16_t* const* w_down, const float* prob_perm, uint16_t* yp,
                    const moe_saved* saved, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * grouped_mlp_fwd_gather -- grouped_mlp_fwd with the dispatch fused into the
 * quantization of its input: grouped row r is token row src_token[r] of x,
 * read by the MXFP8 (FP8) quantizer straight from x, so the bf16 grouped
 * copy xp is never written or read.
 * [BioNeMo, "GroupedLinear": the fused path removes the intermediate data
 *  movement between the permutation and the quantized grouped GEMM;
 *  AutoModel, "专家并行": tokens are sent to the experts that compute them.]
 *
 * Results, saved tensors and workspace contents are bit for bit those of
 * grouped_mlp_fwd on xp[r] = x[src_token[r]] (FP8: the tensor maximum is
 * taken over the gathered rows).
 * precision    MOE_MXFP8 or MOE_FP8 (MOE_BF16: MOE_ERR_ARG; its GEMMs read
 *              xp itself, from moe_permute).
 * x            bf16 [T, H] token rows.
 * src_token    int32 [rows] device, from moe_route; every entry a valid row
 *              of x (not checked).
 * Other arguments and the workspace size: as grouped_mlp_fwd.  prob_perm
 * comes from moe_permute with x = xp = NULL.
 */
int grouped_mlp_fwd_gather(int precision, int E, int H, int I, int64_t rows, const uint16_t* x,
                           const int32_t* src_token, const int32_t* split_sizes,
                           const uint16_t* const* w_gate_up, const uint16_t* const* w_down,
                           const float* prob_perm, uint16_t* yp, const moe_saved* saved,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * grouped_mlp_bwd -- backward of grouped_mlp_fwd.
 * [BioNeMo, "MXFP8与融合MLP": the fused forward has a matching fused backward.]
 *
 * Per expert e (g, u from the saved bf16 A1; s = silu(g), sig = sigmoid(g)):
 *   dA2 = dyp_e W2_e (fp32);  dW2_e = dyp_e^T A2_e
 *   dg = dA2 p u sig (1 + g (1 - sig)),  du = dA2 p s,  dprob = sum_i dA2 s u
 *   dA1 = [dg, du];  dxp_e = dA1 W1_e;  dW1_e = dA1^T xp_e
 * Experts with no rows get exact zeros in dW1_e and dW2_e.  MXFP8 mode
 * quantizes every GEMM operand along that GEMM's contraction axis; FP8 mode
 * casts dyp, the weights (when not saved) and dA1 with one scale per tensor,
 * dA1 after its bf16 materialization.
 *
 * dyp          bf16 [rows, H] (moe_permute of the upstream gradient).
 * xp           as in the forward; read by BF16 mode only (the 8-bit modes
 *              take its columnwise copy from saved) and may be NULL there.
 * split_sizes, w_gate_up, w_down, prob_perm, saved: as in the forward.
 * dxp          bf16 [rows, H] out.
 * dw_gate_up   HOST array of E device pointers, each bf16 [2I, H] out.
 * dw_down      HOST array of E device pointers, each bf16 [H, I] out.
 * dprob_perm   fp32 [rows] out.
 * workspace    moe_workspace_bytes(MOE_OP_MLP_BWD, ...) bytes.
 */
int grouped_mlp_bwd(int precision, int E, int H, int I, int64_t rows, const uint16_t* dyp,
                    const uint16_t* xp, const int32_t* split_sizes,
                    const uint16_t* const* w_gate_up, const uint16_t* const* w_down,
                    const float* prob_perm, const moe_saved* saved, uint16_t* dxp,
                    uint16_t* const* dw_gate_up, uint16_t* const* dw_down, float* dprob_perm,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * grouped_mlp_bwd_gather -- grouped_mlp_bwd with the dispatch of the upstream
 * gradient fused into its quantization: grouped row r of dY is token row
 * src_token[r] of dy.  [The same passages as grouped_mlp_fwd_gather.]
 *
 * Results are bit for bit those of grouped_mlp_bwd on dyp[r] = dy[src_token[r]].
 * precision    MOE_MXFP8 or MOE_FP8 (MOE_BF16: MOE_ERR_ARG).
 * dy           bf16 [T, H] upstream gradient per token.
 * src_token    int32 [rows] device, from moe_route (not checked).
 * Other arguments and the workspace size: as grouped_mlp_bwd (no xp).
 */
int grouped_mlp_bwd_gather(int precision, int E, int H, int I, int64_t rows, const uint16_t* dy,
                           const int32_t* src_token, const int32_t* split_sizes,
                           const uint16_t* const* w_gate_up, const uint16_t* const* w_down,
                           const float* prob_perm, const moe_saved* saved, uint16_t* dxp,
                           uint16_t* const* dw_gate_up, uint16_t* const* dw_down,
                           float* dprob_perm, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Workspace bytes for op (MOE_OP_ROUTE: T, E, k used; MLP ops: rows = T*k,
 * H, I, E, precision used).  Returns 0 for an invalid op.
 */
size_t moe_workspace_bytes(int op, int64_t T, int H, int I, int E, int k, int precision);

/*
 * Regions of the grouped-MLP workspaces (inspection aid).  After
 * grouped_mlp_fwd / grouped_mlp_bwd have run, these regions hold the MXFP8
 * (or FP8) GEMM operands the calls made, until the next call that uses the
 * same workspace.  The codes are in the row-pair layout described with
 * moe_saved; the scales are the bytes of mxfp8_quantize stored block-major,
 * the order the GEMMs read:
 *   rowwise [rows, C]          expert e's row i at row P_0+..+P_{e-1}+i of a
 *                              [RP, C] row-pair matrix, RP = 32*(ceil(rows/32)
 *                              + E) (P_g = 32*ceil(n_g/32)); scales [C/32][RP]
 *   per-expert weights         expert e's [R, C] row-pair matrix at e*R*C,
 *                              scales block-major [C/32][R] at e*R*C/32
 *   grouped columnwise         as the *_col_codes of moe_saved; scales
 *                              [P_g/32][C] per group
 * The region of MOE_WS_A2_* holds the codes the down GEMM read (rowwise
 * MXFP8 of the ScaledSwiGLU output); *_W1_COL_* and *_W2_COL_* are used
 * only when moe_saved carries no weight copies.
 */
typedef enum moe_ws_region {
    /* MOE_OP_MLP_FWD, MOE_MXFP8 / MOE_FP8 */
    MOE_WS_XP_CODES = 0,          /* [rows, H], blocks along H */
    MOE_WS_XP_SCALES = 1,         /* [H/32][rows] */
    MOE_WS_W1_CODES = 2,          /* E x [2I, H], blocks along H */
    MOE_WS_W1_SCALES = 3,         /* E x [H/32][2I] */
    MOE_WS_W2_CODES = 4,          /* E x [H, I], blocks along I */
    MOE_WS_W2_SCALES = 5,         /* E x [I/32][H] */
    MOE_WS_A2_CODES = 6,          /* [rows, I], blocks along I */
    MOE_WS_A2_SCALES = 7,         /* [I/32][rows] */
    /* MOE_OP_MLP_BWD, MOE_MXFP8 / MOE_FP8 */
    MOE_WS_DYP_CODES = 8,         /* [rows, H], blocks along H */
    MOE_WS_DYP_SCALES = 9,        /* [H/32][rows] */
    MOE_WS_DYP_COL_CODES = 10,    /* grouped columnwise [H, P_e] per expert */
    MOE_WS_DYP_COL_SCALES = 11,   /* [P_e/32][H] per expert */
    MOE_WS_W2_COL_CODES = 12,     /* E x [I, H]: W2 blocked along H */
    MOE_WS_W2_COL_SCALES = 13,    /* E x [H/32][I] */
    MOE_WS_W1_COL_CODES = 14,     /* E x [H, 2I]: W1 blocked along 2I */
    MOE_WS_W1_COL_SCALES = 15,    /* E x [2I/32][H] */
    MOE_WS_DA1_CODES = 16,        /* [rows, 2I], blocks along 2I */
    MOE_WS_DA1_SCALES = 17,       /* [2I/32][rows] */
    MOE_WS_DA1_COL_CODES = 18,    /* grouped columnwise [2I, P_e] per expert */
    MOE_WS_DA1_COL_SCALES = 19    /* [P_e/32][2I] per expert */
} moe_ws_region;

/* Byte offset and size of `region` inside the workspace of `op`
 * (MOE_OP_MLP_FWD or MOE_OP_MLP_BWD) for these sizes.  Returns MOE_OK,
 * MOE_ERR_ARG when the op/precision has no such region, MOE_ERR_SHAPE for
 * sizes out of range, or MOE_ERR_NULL. */
int moe_workspace_region(int op, int region, int64_t rows, int H, int I, int E, int precision,
                         size_t* offset, size_t* bytes);

/*
 * grouped_linear_fwd -- one linear map per expert over the expert's rows, all
 * experts in one launch: y_e = x_e W_e^T (no bias), fp32 accumulation,
 * rounded to bf16.
 * [BioNeMo, "GroupedLinear": a grouped linear layer takes the tokens of all
 *  local experts with split_sizes and applies each expert's own weight in one
 *  grouped GEMM instead of one launch per expert.]
 *
 * precision    MOE_BF16 or MOE_MXFP8 (x and W quantized along K first).
 * E            experts, 1..64.   N: out_features, K: in_features, both
 *              multiples of 32, with N * K * 2 and max(N, K)/32 *
 *              32*(ceil(rows/32) + E) below 2^31 (otherwise MOE_ERR_SHAPE).
 * rows         total rows (sum of split_sizes), 0 <= rows <= INT32_MAX.
 * x            bf16 [rows, K], expert-grouped.   split_sizes: int32 [E] device.
 * w            HOST array of E device pointers, each bf16 [N, K].
 * y            bf16 [rows, N] out.
 * workspace    moe_workspace_bytes(MOE_OP_LINEAR_FWD, rows, K, N, E, 1, precision).
 */
int grouped_linear_fwd(int precision, int E, int N, int K, int64_t rows, const uint16_t* x,
                       const int32_t* split_sizes, const uint16_t* const* w, uint16_t* y,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * grouped_linear_bwd -- backward of grouped_linear_fwd: dx_e = dy_e W_e and
 * dW_e = dy_e^T x_e (contraction over the expert's rows; exact zeros for an
 * expert with no rows), fp32 accumulation, rounded to bf16.  MXFP8 mode
 * quantizes dy along N and W along N for dx, and dy and x in 32-row blocks
 * that restart at each expert's first row for dW.
 * dy           bf16 [rows, N].   x: bf16 [rows, K] (used for dW).
 * dx           bf16 [rows, K] out, or NULL (not computed).
 * dw           HOST array of E device pointers, each bf16 [N, K] out, or
 *              NULL (not computed).
 * Other arguments as grouped_linear_fwd; workspace of
 * moe_workspace_bytes(MOE_OP_LINEAR_BWD, rows, K, N, E, 1, precision) bytes.
 */
int grouped_linear_bwd(int precision, int E, int N, int K, int64_t rows, const uint16_t* dy,
                       const uint16_t* x, const int32_t* split_sizes, const uint16_t* const* w,
                       uint16_t* dx, uint16_t* const* dw, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);


/*
 * Launch trace (measurement aid).  moe_trace_enable(capacity) creates, once,
 * 2*capacity HIP events and starts recording: every kernel launch made by the
 * calls above is then bracketed by a start and a stop event recorded on the
 * launch's stream (at most `capacity` launches; later ones are not traced).
 * After the stream has passed them, moe_trace_read(i, &name, &ms) returns the
 * i-th launch's kernel name (static string) and duration.  Enabling again
 * resets the count.  moe_trace_filter(prefix) restricts the trace to launches
 * whose name starts with prefix (NULL or "" = every launch; it stays set until
 * changed): each traced launch adds two event records to its stream, so a
 * timed loop traces only the kernels it reports.  Not for concurrent use from
 * several host threads.
 * Returns MOE_OK, MOE_ERR_ARG (bad capacity/index) or MOE_ERR_HIP.
 */
void moe_trace_filter(const char* prefix);
int moe_trace_enable(int capacity);
void moe_trace_disable(void);
int moe_trace_count(void);
int moe_trace_read(int i, const char** name, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */

/*
 * libattn: fused exact-attention forward for AMD MI355X (gfx950).
 *
 * C ABI. Plain pointers and sizes only; no framework types cross it.
 *
 * The operation, per batch b and head h, with Q of shape (Nq, d) and K, V of
 * shape (Nkv, d) (Nq = Nkv = N for self-attention):
 *
 *     O = softmax(scale * Q K^T + mask) V
 *     LSE = log(rowsum(exp(scale * Q K^T + mask)))   (optional, attn_fwd_ex)
 *
 * as defined by the AWS Neuron NKI tutorial "Fused Self Attention"
 * (section "Background": S = Q K^T, R = softmax(S) V over (seqlen, d_head)
 * tensors in bfloat16), with the 1/sqrt(d) scale and the -inf causal mask of
 * "Profiling in PyTorch" part 3 (section "Deconstructing Naive Attention"),
 * and the wrap-around 2D neighbourhood window requested in NATTEN issue 142
 * (a window that wraps circularly at the grid's edges; its 5x5 grid, kernel
 * size 3 example).
 *
 * The N x N score matrix is never written to memory: scores are produced
 * tile by tile, reduced with a running row maximum and row sum, and divided
 * once after the product with V (NKI tutorial, section "Softmax
 * implementation"; PhotoRoom's xformers post, the running-softmax
 * paragraph).
 *
 * Types at the boundary: every `stream` argument is a `void*` that holds a
 * hipStream_t (NULL = the default stream), so that this header needs no HIP
 * include; functions return attn_status_t; attn_status_string takes an
 * int32_t so that any integer, including a code this version does not know,
 * can be passed to it.
 *
 * State: the library keeps no per-call state. It caches two read-only facts
 * per device the first time a call needs them (the CU count, used to plan
 * the remainder split and the causal dispatch order, and the device address
 * of attn_fwd_ex_static's scratch array); the caches are filled under a lock
 * or an atomic store and never change afterwards.
 */
#ifndef LIBATTN_ATTN_H
#define LIBATTN_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 6: the split workspace of attn_fwd_ws / attn_fwd_ex also holds one arrival
 * counter per split tile (its size grew by at most 1 KB), and ATTN_STATIC_SCRATCH_BYTES
 * with it; signatures are unchanged. */
#define ATTN_ABI_VERSION 6

/* Mask modes. */
typedef enum {
    ATTN_MASK_NONE = 0,   /* every key visible to every query */
    ATTN_MASK_CAUSAL = 1, /* key j visible to query i iff j <= i ("Profiling in PyTorch",
                             the naive causal module and SDPA's is_causal=True; with
                             Nq != Nkv this is SDPA's top-left alignment) */
    ATTN_MASK_NA2D = 2,   /* 2D neighbourhood window over a row-major token grid
                             (NATTEN issue 142); parameters in attn_na2d_params_t */
    ATTN_MASK_NA3D = 3    /* 3D neighbourhood window over a row-major token volume (the MR
                             volumes of NATTEN issue 142); parameters in attn_na3d_params_t */
} attn_mask_mode_t;

/*
 * 2D neighbourhood parameters (host memory, read during the call only).
 *
 * Token n sits at grid row y = n / grid_w and column x = n % grid_w;
 * grid_h * grid_w must equal N (and queries and keys must be equally many).
 * Along each axis, with r = kernel / 2 and dilation dil >= 1:
 *   wrap = 1: key allowed when its coordinate is (c + dil * t) mod L for some
 *             t in -r..r, c the query's coordinate (a centred window that wraps
 *             at the borders like a convolution with circular padding; NATTEN
 *             issue 142, the 5x5 example and the 1D recipe that pads by
 *             kernel / 2 * dilation). Requires (kernel - 1) * dil < L, so each
 *             key counts once.
 *   wrap = 0: the standard window: among the cells congruent to c mod dil,
 *             the `kernel` consecutive ones starting at clamp(i - r, 0, L_g -
 *             kernel), where i is the query's index among them and L_g their
 *             number, i.e. shifted inside the grid at the edges (NATTEN issue
 *             142, the replies on window_start and window_end and on clamping
 *             the window to the edges). Requires kernel * dil <= L.
 * A key is visible when both axes allow it. Kernels must be odd and >= 1.
 */
typedef struct {
    int32_t grid_h, grid_w;
    int32_t kernel_h, kernel_w;
    int32_t wrap_h, wrap_w;  /* 1 = circular, 0 = clamped */
    int32_t dil_h, dil_w;    /* dilation, >= 1 */
} attn_na2d_params_t;

/*
 * 3D neighbourhood parameters (host memory, read during the call only).
 * Token n sits at depth z, row y and column x with
 * n = (z * grid_h + y) * grid_w + x; grid_d * grid_h * grid_w must equal N.
 * Each axis follows the rules of attn_na2d_params_t; a key is visible when
 * all three axes allow it.
 */
typedef struct {
    int32_t grid_d, grid_h, grid_w;
    int32_t kernel_d, kernel_h, kernel_w;
    int32_t wrap_d, wrap_h, wrap_w;
    int32_t dil_d, dil_h, dil_w;
} attn_na3d_params_t;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, non-finite scale, unknown
                                 mask mode, params given when not a neighbourhood mode,
                                 o or lse overlapping an input or each other */
    ATTN_ERR_UNSUPPORTED = 2, /* head size d other than 32, 64 or 128, or a problem too large
                                 for 32-bit launch geometry */
    ATTN_ERR_PARAMS = 3,      /* neighbourhood parameters inconsistent (grid size != Nq or
                                 != Nkv, even or out-of-range kernel, wrap not 0/1,
                                 dilation < 1, window too large for its axis) */
    ATTN_ERR_ALIGNMENT = 4,   /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
    ATTN_ERR_HIP = 5,         /* the HIP runtime reported an error (no device, a failed
                                 device query, or a failed launch) */
    ATTN_ERR_WORKSPACE = 6,   /* attn_fwd_ws: workspace NULL, smaller than
                                 attn_fwd_workspace_size, not 256-byte aligned, or
                                 overlapping q, k, v or o */
    ATTN_ERR_SCRATCH = 7      /* attn_fwd_ex_static: the problem's split needs more than
                                 ATTN_STATIC_SCRATCH_BYTES */
} attn_status_t;

/*
 * attn_fwd: O = softmax(scale * Q K^T + mask) V, asynchronously on `stream`.
 *
 * q, k, v : device pointers, bfloat16, contiguous [B, H, N, d] (d fastest),
 *           16-byte aligned; read only.
 * o       : device pointer, bfloat16, contiguous [B, H, N, d], 16-byte
 *           aligned; written with the result rounded to nearest even. Must
 *           not overlap q, k or v.
 * B, H, N : batch, heads, tokens (> 0). Queries and keys share N.
 * d       : head size, 32, 64 or 128.
 * scale   : finite multiplier applied to Q K^T before the mask (0 and
 *           negative values are legal; scale = 0 averages V over the
 *           visible keys).
 * mask_mode : an attn_mask_mode_t value.
 * params  : NULL unless mask_mode is ATTN_MASK_NA2D or ATTN_MASK_NA3D, then a
 *           host pointer to an attn_na2d_params_t or attn_na3d_params_t.
 * stream  : a hipStream_t (NULL = the default stream).
 *
 * The caller owns all memory. The library allocates nothing, keeps no state
 * between calls (beyond the per-device caches above), never synchronises and
 * is safe to call concurrently on different streams. Exactly one kernel is
 * launched per call.
 *
 * Returns ATTN_OK after the launch is queued. Argument errors are detected
 * before any device work and leave o untouched. ATTN_ERR_HIP reports a
 * launch failure; o is then undefined.
 */
attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o,
                       int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                       int32_t mask_mode, const void* params, void* stream);

/*
 * attn_fwd_ws: the same operation and arguments as attn_fwd, plus a device
 * workspace that lets unmasked problems spread evenly over the whole chip.
 * (attn_fwd_ex is the same call with Nq, Nkv and the optional lse output.)
 *
 * One work-group per query tile of 128 queries leaves the GPU unevenly
 * loaded when the tile count is not a multiple of the CU count (for example
 * 320 tiles on 256 CUs: 64 CUs do two tiles, 192 do one). For unmasked
 * problems of fewer than two tiles per CU, this entry point keeps one
 * work-group per tile for a whole round of tiles and cuts each remaining
 * tile along its keys into parts that run beside them, so every CU does
 * about the same work; the last part of each such tile to finish combines
 * the parts exactly (the running-softmax rescaling of PhotoRoom's xformers
 * post, running-softmax paragraph, applied between parts) and stores the
 * tile. The parts meet through one arrival counter per split tile in the
 * workspace, which a one-work-group kernel queued on the same stream just
 * before zeroes. The result equals attn_fwd's up to floating-point summation
 * order, and does not depend on which part finishes last.
 * Other problems (causal and neighbourhood masks, tile counts that fill
 * the chip for two or more rounds, or that would cut a tile into parts of
 * fewer than 2 key tiles) run exactly as attn_fwd with one kernel, and the
 * workspace is then not touched (it may be NULL when
 * attn_fwd_workspace_size gives 0).
 *
 * workspace       : device scratch memory of at least attn_fwd_workspace_size
 *                   bytes for this problem, 256-byte aligned, disjoint from
 *                   q, k, v and o; any initial content. Owned by the caller.
 *                   Calls that share a workspace must not run concurrently
 *                   (queue them on one stream).
 * workspace_bytes : its size in bytes.
 *
 * The size depends on the current device (its CU count) and the head size;
 * it is at most the CU count x 18, 34 or 66 KB for d = 32, 64 or 128, plus
 * 4 bytes per split tile rounded up to 256 (about 8.9 MB at d = 64 on an
 * MI355X). Returns the codes of attn_fwd, and
 * ATTN_ERR_WORKSPACE for a workspace that does not meet the above; all
 * argument errors are detected before any device work.
 * The library still allocates nothing.
 */
attn_status_t attn_fwd_ws(const void* q, const void* k, const void* v, void* o,
                          int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                          int32_t mask_mode, const void* params, void* workspace,
                          uint64_t workspace_bytes, void* stream);

/*
 * attn_fwd_workspace_size: bytes of workspace that attn_fwd_ws needs for
 * this problem on the current HIP device, written to *bytes (0 when the
 * problem runs without parts). Checks the sizes, mask and parameters like
 * attn_fwd_check (the scale is not an argument); ATTN_ERR_INVALID_ARG if
 * bytes is NULL, ATTN_ERR_HIP if there is no usable device.
 */
attn_status_t attn_fwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d,
                                      int32_t mask_mode, const void* params,
                                      uint64_t* bytes);

/*
 * attn_fwd_check: the argument checks of attn_fwd alone, for a problem with
 * the given sizes, scale, mask and parameters; no device work is done and
 * no pointer is dereferenced (pointer checks are not part of it). Returns
 * the status attn_fwd would return for valid, aligned, non-overlapping
 * pointers.
 */
attn_status_t attn_fwd_check(int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                             int32_t mask_mode, const void* params);

/*
 * attn_fwd_ex: the general form of attn_fwd_ws.
 *
 *     O = softmax(scale * Q K^T + mask) V,  LSE = log(sum_j exp(scale * (Q K^T)_ij + mask_ij))
 *
 * q       : device, bfloat16 [B, H, Nq, d]; k, v: device, bfloat16 [B, H, Nkv, d]
 *           (cross-attention when Nq != Nkv); o: device, bfloat16 [B, H, Nq, d].
 *           Contiguous, 16-byte aligned; o disjoint from q, k and v.
 * lse     : NULL, or a device pointer to float32 [B, H, Nq], 4-byte aligned,
 *           disjoint from q, k, v, o and the workspace: receives each row's
 *           natural-log logsumexp of the scaled, masked scores (the statistic a
 *           backward pass recomputes the probabilities from; NATTEN issue 142's
 *           fused forward saves it beside the output). -inf for a row with no
 *           visible key (not reachable with these masks).
 * Nq, Nkv : query and key counts (> 0). The neighbourhood masks need Nq = Nkv.
 * d       : 32, 64 or 128.
 * Other arguments, the workspace rules and the errors are those of
 * attn_fwd_ws, with Nq and Nkv in place of N; the workspace size comes from
 * attn_fwd_ex_workspace_size.
 */
attn_status_t attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                          int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, float scale,
                          int32_t mask_mode, const void* params, void* workspace,
                          uint64_t workspace_bytes, void* stream);

/* attn_fwd_workspace_size for attn_fwd_ex's problem (Nq queries, Nkv keys). */
attn_status_t attn_fwd_ex_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d,
                                         int32_t mask_mode, const void* params, uint64_t* bytes);

/* attn_fwd_check for attn_fwd_ex's problem (Nq queries, Nkv keys). */
attn_status_t attn_fwd_ex_check(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, float scale,
                                int32_t mask_mode, const void* params);

/*
 * attn_fwd_ex_static: attn_fwd_ex for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid it).
 * The same computation, kernels and results as attn_fwd_ex, but the split
 * workspace is a static device array inside the library (one per device, of
 * ATTN_STATIC_SCRATCH_BYTES, held until the process ends) instead of a caller
 * buffer; no call allocates or frees memory. The array needs no initial content
 * and keeps the last call's parts. Every call on a device shares that device's
 * array: calls that overlap on one device (concurrent streams, or host threads
 * with the same device current) race and give undefined outputs; order them on
 * one stream. Problems whose split needs more than the array (none on devices of
 * up to 256 CUs) fail with ATTN_ERR_SCRATCH before any device work; other errors
 * are those of attn_fwd_ex.
 */
#define ATTN_STATIC_SCRATCH_BYTES 17302528  /* 256 part slots of the d = 128 kernel + 256 counters */
attn_status_t attn_fwd_ex_static(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, float scale,
                                 int32_t mask_mode, const void* params, void* stream);

/*
 * attn_bwd: the backward pass of attn_fwd_ex. For the output gradient dO it
 * writes the gradients of O = softmax(scale * Q K^T + mask) V:
 *
 *     dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale * dS K,  dK = scale * dS^T Q,
 *
 * with P = exp(scale * Q K^T + mask - LSE) recomputed from the forward's
 * logsumexp and D the row sums of dO * O (NATTEN issue 142: the fused forward
 * saves the logsumexp for its autograd backward).
 *
 * q, k, v : the forward's inputs (device, bfloat16, [B,H,Nq,d] and [B,H,Nkv,d]).
 * o, lse  : the forward's output and logsumexp from attn_fwd_ex (lse float32
 *           [B,H,Nq], 4-byte aligned).
 * dout    : dO, device bfloat16 [B,H,Nq,d].
 * dq, dk, dv : outputs, device bfloat16 shaped like q, k and v, rounded to
 *           nearest even; disjoint from every input and from each other.
 * mask_mode, params : as for attn_fwd_ex (no mask, causal, 2D or 3D
 *           neighbourhood windows with wrap, clamp and dilation); d = 32, 64
 *           or 128, as for the forward.
 * workspace : device memory of at least attn_bwd_workspace_size bytes
 *           (B*H*Nq float32 row sums), 256-byte aligned, disjoint from the
 *           tensors; any content; calls sharing it must not overlap.
 * The other arguments and the error rules are those of attn_fwd_ex. Two
 * kernels are queued on `stream` (the first also leaves D in the workspace for
 * the second); the library allocates nothing.
 */
attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Nq,
                       int64_t Nkv, int64_t d, float scale, int32_t mask_mode, const void* params,
                       void* workspace, uint64_t workspace_bytes, void* stream);

/* Bytes of workspace attn_bwd needs (B * H * Nq * 4), after the argument checks
 * of attn_bwd that need no pointer. */
attn_status_t attn_bwd_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d,
                                      int32_t mask_mode, const void* params, uint64_t* bytes);

/* A static, human-readable description of a status code (never NULL). */
const char* attn_status_string(int32_t status);

/* ATTN_ABI_VERSION of the built library. */
int32_t attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_ATTN_H */

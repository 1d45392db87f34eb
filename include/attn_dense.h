/*
 * attn_dense.h - C ABI of the MI355X (gfx950) dense attention library.
 *
 * Operations (page "Audit SGLang interfaces and refresh validated kernel solutions"):
 *   - definitions/dense_attention/noncausal_dense_attention_h32_d128.json and
 *     ..._h32_d64.json: O = softmax(Q K^T * D^-0.5) V per batch and head, noncausal,
 *     no mask, no dropout, FP32 accumulation, BF16 output. Self attention has Nq = Nk;
 *     the description also admits cross attention with Nq != Nk.
 *   - definitions/block_causal_attention/prefix_cached_block_causal_h32_d128.json
 *     (post-change text): each query attends to every key of the concatenation of
 *     K_prefix then K_current along the sequence axis, with V_prefix then V_current.
 *     The operand order Q, K_prefix, V_prefix, K_current, V_current is the pages'
 *     positional order (same page, interfaces.json entry for that definition).
 * The scale is not an argument: the pages fix it to head_dim ** -0.5 (same page,
 * README "Feasible changes" and the definitions' descriptions).
 *
 * Conventions shared by every entry point:
 *   - Tensors are contiguous [B, N, H, D] arrays of BF16 (raw 16-bit patterns) in
 *     device memory of the current HIP device. N is Nq for Q and the output, Nk / Np /
 *     Nq for the key and value operands as stated per call.
 *   - Every pointer must be 16-byte aligned (the kernels use 128-bit accesses).
 *   - D must be 64 or 128. H, B and the sequence lengths must be >= 1 (Np >= 0).
 *     The pages fix H = 32; any H >= 1 is accepted.
 *   - Ownership: the caller owns all buffers. Inputs are read only and never written.
 *     The output is caller-allocated and must not overlap any input.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL means the null stream) and the
 *     call returns without waiting. Device-side faults surface at the caller's next
 *     synchronisation. Results are deterministic: the same inputs and the same launch
 *     plan give the same bits.
 *   - Return value: ATTN_OK (0) or a negative ATTN_ERR_* code. All argument checks run
 *     before any work is enqueued (the only HIP call before them asks for the current
 *     device), so an invalid call touches no device state. No exception crosses the ABI.
 *   - Work space (split-KV partial results when the grid would underfill the GPU, and
 *     the image-id summaries of attn_block_causal), per device, from one of two sources:
 *       * the caller's buffer, if attn_set_workspace() gave one for the current device:
 *         used as is, never grown or freed; a call that needs more returns
 *         ATTN_ERR_WORKSPACE, a buffer overlapping the call's tensors ATTN_ERR_ALIAS;
 *       * otherwise the library's own buffer, allocated with hipMalloc when a call
 *         needs more than it holds (at least doubling). A superseded buffer is never
 *         freed (launches in flight and HIP graphs captured earlier keep using it), so
 *         growing never synchronises the device. Allocation is not allowed during HIP
 *         graph capture: callers that capture reserve the space first, with
 *         attn_reserve_workspace() or one uncaptured call of the same shape, or supply
 *         their own buffer.
 *     Every call that uses the work space on a device shares that one buffer: such
 *     calls must not run at the same time on different streams of one device (order
 *     them on one stream, or give each stream its own buffer through
 *     attn_set_workspace() before its calls); calls on one stream are ordered by it.
 */
#ifndef ATTN_DENSE_H
#define ATTN_DENSE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK 0
#define ATTN_ERR_NULL (-1)        /* a required pointer is NULL */
#define ATTN_ERR_SHAPE (-2)       /* B, N, H < 1, or Np < 0 */
#define ATTN_ERR_UNSUPPORTED (-3) /* D not in {64, 128}, or a bad launch option */
#define ATTN_ERR_ALIGN (-4)       /* a pointer is not 16-byte aligned */
#define ATTN_ERR_ALIAS (-5)       /* the output (or a caller's work space) overlaps an input */
#define ATTN_ERR_OVERFLOW (-6)    /* a size exceeds the index range of the kernels */
#define ATTN_ERR_WORKSPACE (-7)   /* the work space could not be allocated or is too small */
#define ATTN_ERR_HIP (-8)         /* a HIP runtime call or kernel launch failed */

/*
 * Dense noncausal self attention (Nq = Nk = N).
 * q, k, v: [B, N, H, D] BF16 inputs. out: [B, N, H, D] BF16 output.
 * stream: hipStream_t to enqueue on.
 */
int attn_dense(const void* q, const void* k, const void* v, void* out, int B, int N, int H,
               int D, void* stream);

/*
 * Prefix-cached attention: Q attends to every key of (K_prefix ++ K_current).
 * q: [B, Nq, H, D]; kp, vp: [B, Np, H, D]; kc, vc: [B, Nq, H, D]; out: [B, Nq, H, D].
 * The pages require Np >= 1; Np = 0 is also accepted and equals
 * attn_dense(q, kc, vc) (kp and vp may then be NULL).
 */
int attn_prefix(const void* q, const void* kp, const void* vp, const void* kc, const void* vc,
                void* out, int B, int Nq, int Np, int H, int D, void* stream);

/*
 * Dense noncausal cross attention (Nq != Nk allowed by the definitions' description).
 * q: [B, Nq, H, D]; k, v: [B, Nk, H, D]; out: [B, Nq, H, D].
 */
int attn_cross(const void* q, const void* k, const void* v, void* out, int B, int Nq, int Nk,
               int H, int D, void* stream);

/*
 * Block-causal attention without a prefix (page "Audit SGLang interfaces and refresh
 * validated kernel solutions",
 * definitions/block_causal_attention/prefix_cached_block_causal_h32_d128_prefix0.json,
 * post-change text; operand order Q, K_current, V_current, image_ids): query i sees
 * key j when j <= i, or when image_ids[i] >= 0 and image_ids[j] == image_ids[i]
 * (text tokens carry -1; the pages describe nonnegative ids as contiguous image
 * blocks, but any ids are handled exactly). Scale D^-0.5.
 * q, k, v: [B, N, H, D] BF16; image_ids: [N] int32 in device memory, shared by the
 * batch, 16-byte aligned; out: [B, N, H, D] BF16, must overlap no input.
 * Uses the device's work space (16 bytes per 32 rows) for summaries of the ids.
 */
int attn_block_causal(const void* q, const void* k, const void* v, const int* image_ids,
                      void* out, int B, int N, int H, int D, void* stream);

/*
 * 3-D neighborhood attention (page "Audit SGLang interfaces and refresh validated kernel
 * solutions", definitions/neighborhood_attention/neighborhood_attention_3d_*: the call
 * natten.functional.na3d(q, k, v, kernel_size=(kt, ky, kx), scale=1.0); the model's
 * scale is already in Q).
 *   q, k, v, out: [B, T, Y, X, H, D] BF16, contiguous, device memory, D = 64.
 *   Query (b, t, y, x, h) attends to the keys (b, t', y', x', h) with t' in the window of
 *   t on the T axis (odd size kt, centred on t and moved inside [0, T) at the ends:
 *   start = max(0, min(t - kt/2, T - kt))), likewise y' on Y with ky and x' on X with
 *   kx: exactly kt*ky*kx keys each. Scores are plain dot products (scale 1); softmax in
 *   FP32, output rounded to BF16. The neighborhood is NATTEN's published one; the pages
 *   name na3d without defining it.
 * Errors: ATTN_ERR_SHAPE for a size < 1 or a window that is even or longer than its
 * axis; ATTN_ERR_UNSUPPORTED for D != 64 or kx > 17; ATTN_ERR_OVERFLOW, ATTN_ERR_ALIGN,
 * ATTN_ERR_ALIAS as for the other calls. No work space.
 */
int attn_na3d(const void* q, const void* k, const void* v, void* out, int B, int T, int Y,
              int X, int H, int D, int kt, int ky, int kx, void* stream);

/*
 * General form behind the dense, prefix and cross calls, with explicit launch options.
 * The keys are segment 0 (k0/v0, n0 rows) followed by segment 1 (k1/v1, n1 rows);
 * n0 + n1 >= 1, and a segment with zero rows may have NULL pointers.
 * num_splits: 0 = automatic, otherwise the number of key ranges computed in parallel
 *             and merged by a combine step (clamped to the number of key tiles).
 * waves:      0 = automatic, otherwise 2, 4 or 8 wavefronts (32 query rows each)
 *             per workgroup; 8 selects the ping-pong schedule (two wave groups
 *             alternating matrix and softmax phases).
 * Results for any options agree with each other up to floating-point rounding.
 */
int attn_fwd_ex(const void* q, const void* k0, const void* v0, int n0, const void* k1,
                const void* v1, int n1, void* out, int B, int Nq, int H, int D, int num_splits,
                int waves, void* stream);

/*
 * attn_fwd_ex without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and errors as attn_fwd_ex, except for the split-KV work
 * space: it is a static device array of 64 MiB (67108864 bytes) that the library holds
 * on every GPU it runs on until the process ends, never the library's or the caller's
 * work space above. A plan that needs more (attn_plan's workspace_bytes) returns
 * ATTN_ERR_WORKSPACE before any work is enqueued. Every call on one GPU shares that
 * array: calls that may overlap in time on one GPU (different streams, or graphs
 * replayed concurrently) race and must be ordered by the caller. No call here
 * allocates, frees or synchronises.
 */
int attn_fwd_ex_noalloc(const void* q, const void* k0, const void* v0, int n0, const void* k1,
                        const void* v1, int n1, void* out, int B, int Nq, int H, int D,
                        int num_splits, int waves, void* stream);

/*
 * Launch plan the library would use for a call, computed on the host only (no HIP
 * call). Any output pointer may be NULL. Returns ATTN_OK or a shape/size error.
 *   splits:          key ranges computed in parallel (1 = no combine step)
 *   waves:           wavefronts per workgroup
 *   workgroups:      workgroups of the main kernel
 *   workspace_bytes: split-KV work space needed (0 when splits == 1)
 */
int attn_plan(int B, int Nq, int Nk, int H, int D, int num_splits, int waves, int* splits,
              int* waves_out, long long* workgroups, long long* workspace_bytes);

/*
 * Launch plan of attn_na3d for these sizes and window, computed on the host only (no
 * HIP call). Any output pointer may be NULL. Returns ATTN_OK or the size/window error
 * attn_na3d would return.
 *   query_cols: positions on X of a wavefront's query tile (16, 8 or 4; the tile is
 *               32 / query_cols rows y by query_cols positions), chosen per window with
 *               its key blocks of 32 keys (32 positions of one row for 16; 16 positions
 *               of two rows for 8; for 4, 16 positions of two rows or, when kx <= 5 and
 *               8 * X * H * D < 2^32, 8 positions of four rows)
 *   workgroups: workgroups of the kernel (four wavefronts each: 1, 2 or 4 frames by 4, 2
 *               or 1 row tiles, whichever walks the fewest key blocks)
 */
int attn_na3d_plan(int B, int T, int Y, int X, int H, int D, int kt, int ky, int kx,
                   int* query_cols, long long* workgroups);

/*
 * Makes sure the current device's work space holds at least `bytes`: grows the
 * library's buffer if it is smaller (no device synchronisation), or, when the caller
 * supplied the buffer, checks that it is large enough. Returns ATTN_OK,
 * ATTN_ERR_WORKSPACE (allocation failed, or the caller's buffer is too small) or
 * ATTN_ERR_HIP (no current device).
 */
int attn_reserve_workspace(long long bytes);

/*
 * Caller-supplied work space for the current device (the pages keep engine set-up
 * such as work spaces out of the timed call: page "SGLang interface and
 * implementation audit - 2026-10-19", section "Validation and timing").
 *   ptr:   device memory of the current device, 256-byte aligned, `bytes` long; the
 *          caller owns it and must keep it allocated while calls that use it may still
 *          run (including replays of HIP graphs captured with it). NULL reverts to the
 *          library's own buffer.
 *   bytes: its size; attn_plan() reports what a call needs (workspace_bytes), and a
 *          block-causal call needs 16 bytes per 32 rows.
 * Later calls on this device, from any thread, use it until the next
 * attn_set_workspace(). Returns ATTN_OK, ATTN_ERR_ALIGN (ptr not 256-byte aligned),
 * ATTN_ERR_SHAPE (bytes < 0) or ATTN_ERR_HIP (no current device).
 */
int attn_set_workspace(void* ptr, long long bytes);

/* Static description of an error code (never NULL). */
const char* attn_strerror(int code);

/* ABI version of this header: 1. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DENSE_H */

/*
 * msda.h -- C ABI of the MI355X (gfx950) multi-scale deformable attention
 * (MSDeformAttn) sampling core.
 *
 * The operation.  For every batch b, query q and head m the core returns
 *
 *     out[b, q, m*D + d] = sum_l sum_k A[b,q,m,l,k] * S_l(value[b, :, m, d], loc[b,q,m,l,k])
 *
 * the attention-weighted sum over levels l and points k of bilinear samples of
 * the flattened multi-level value ("Deformable attention: multi-scale sparse
 * sampling and detection practice", section 2.2, the multi-scale formula with
 * the value and output projections left outside; "Deformable DETR" tutorial,
 * section 3.3).  A sample S_l at normalized location (u, v) of level l, whose
 * rows in the level table are (H_l, W_l) and whose pixels start at flattened
 * index start_l, takes the pixel coordinates x = u*W_l - 0.5, y = v*H_l - 0.5
 * (the grid_sample convention with align_corners=False, first page, sections
 * 2.3 and 3.2) and sums the four integer neighbours (x0,y0), (x0+1,y0),
 * (x0,y0+1), (x0+1,y0+1) with bilinear weights; neighbours outside the map
 * contribute zero (first page, section 2.3).  The pixel coordinate is
 * computed as one fp32 fused multiply-add and floored in fp32.  Locations
 * whose coordinates are not finite contribute zero.
 *
 * Pixel convention.  With the flag MSDA_ALIGN_CORNERS (forward and backward
 * alike) the pixel coordinates are instead x = u*(W_l - 1), y = v*(H_l - 1),
 * one fp32 rounding of the product: grid_sample's align_corners=True, which
 * the first page (section 2.3) advises offering as a configuration option
 * because the two conventions differ by half a pixel, and which its section 6
 * notes some inference engines use by default.  The location gradients then
 * carry the factors W_l - 1 and H_l - 1 instead of W_l and H_l.
 *
 * Layouts.  Every tensor is dense and row-major with no strides:
 *   value              [B, Nv, M, D]          fp32, or bf16 when value_dtype == MSDA_BF16
 *   spatial_shapes     [L, 2]  int64, rows (H_l, W_l)
 *   level_start_index  [L]     int64, start_l = sum of H*W of the levels before l
 *   sampling_loc       [B, Nq, M, L, K, 2]    fp32, last axis (x, y) = (u, v), normalized
 *   attn_weight        [B, Nq, M, L, K]       fp32
 *   out, grad_out      [B, Nq, M*D]           fp32, head-major (channel m*D + d)
 *   grad_value         [B, Nv, M, D]          fp32 for either value dtype
 *   grad_sampling_loc  [B, Nq, M, L, K, 2]    fp32
 *   grad_attn_weight   [B, Nq, M, L, K]       fp32
 * with Nv = sum_l H_l*W_l.
 *
 * Memory and ownership.  Every tensor pointer, spatial_shapes and
 * level_start_index included, is a DEVICE pointer on the current HIP device;
 * the caller allocates and owns all of them, and the backward's scratch
 * workspace too.  The library allocates no memory and keeps no state between
 * calls, except msda_backward_noalloc's static scratch (see there).  Outputs
 * must not alias inputs.  Calls on different streams may run concurrently
 * when each has its own outputs and workspace.
 *
 * Streams and errors.  `stream` is a hipStream_t (NULL = the null stream).
 * Work is enqueued on it and the call returns without synchronizing; a
 * kernel fault therefore surfaces at the caller's next synchronization.
 * The backward entry points can also use a second, caller-owned stream
 * (side_stream, with two caller-created hipEvent_t in side_events[0..1]):
 * the grad_attn_weight / grad_sampling_loc kernel then runs there,
 * concurrently with the grad_value kernels on `stream`, on problems of at
 * least 2^18 sampling points (B * Nq * M * L * K); smaller ones run on
 * `stream` alone, as the fork and join would cost more than they save.
 * When it uses side_stream the call forks it from `stream` (side_events[0])
 * and joins it back into `stream` (side_events[1]) before returning -- on
 * its error paths too -- so work
 * enqueued on `stream` afterwards sees every output complete (this also
 * holds under stream capture).  side_stream NULL (or equal to `stream`):
 * everything runs on `stream`, side_events is ignored.  A side stream and its
 * events must not be used by two calls in flight at once (one set per caller
 * stream).  Priorities other than the default are not needed.
 * Every function returns an msda_status; nothing is thrown across the ABI.
 * The launch-time checks cover null pointers, negative sizes, 1 <= L <= 16,
 * the supported head widths and dtypes, and the 32-bit addressing limit.
 * The level table is on the device and is not read by the host:
 * msda_validate_host checks a host copy of it.  The kernels address value and
 * grad_value through range-checked buffer descriptors, so an inconsistent
 * level table cannot make them touch memory outside those tensors: a level
 * that does not fit inside value contributes zero.
 *
 * Limits.  D in {4, 8, 16, 32, 64, 128, 256}; 1 <= L <= 16; K >= 1;
 * Nv*M*D*4 < 2^31 bytes (one batch slice of grad_value); Nq*M*L*K*2 < 2^31;
 * B*Nq*M*L*K*4 < 2^32.  msda_backward also needs Nq <= 2^25.
 * B, Nq may be 0 (nothing is launched, except the zero fill of grad_value).
 */
#ifndef MSDA_H
#define MSDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum msda_status {
    MSDA_OK = 0,
    MSDA_ERR_NULL = -1,        /* a required pointer is NULL                          */
    MSDA_ERR_SHAPE = -2,       /* sizes are negative or inconsistent                  */
    MSDA_ERR_DTYPE = -3,       /* value_dtype is not an msda_dtype                    */
    MSDA_ERR_UNSUPPORTED = -4, /* valid but outside the limits above (D, L, size)     */
    MSDA_ERR_HIP = -5,         /* the HIP runtime refused a launch (see msda_last_hip_error) */
    MSDA_ERR_WORKSPACE = -6,   /* workspace too small or not 256-byte aligned             */
    MSDA_ERR_SCRATCH = -7      /* msda_backward_noalloc: even the smallest pass needs
                                  more than MSDA_NOALLOC_SCRATCH_BYTES                 */
} msda_status;

typedef enum msda_dtype {
    MSDA_F32 = 0,
    MSDA_BF16 = 1              /* bfloat16 value only; all else fp32                  */
} msda_dtype;

/* Flags (unknown bits give MSDA_ERR_UNSUPPORTED). */
#define MSDA_BWD_ACCUMULATE 1u /* backward: add into grad_value instead of overwriting  */
#define MSDA_ALIGN_CORNERS 2u  /* both: x = u*(W-1), y = v*(H-1) (align_corners=True)   */
#define MSDA_SOFTMAX_PER_LEVEL 4u /* fused entry points: softmax over each level's K points */
#define MSDA_BWD_BINNED 8u     /* backward: the binned grad_value pipeline at any size      */

/*
 * Forward: out = MSDeformAttn core(value, level table, sampling_loc, attn_weight).
 * out is overwritten.  value_dtype is an msda_dtype; flags is 0 or
 * MSDA_ALIGN_CORNERS.
 */
msda_status msda_forward(const void *value, int value_dtype,
                         const int64_t *spatial_shapes, const int64_t *level_start_index,
                         const float *sampling_loc, const float *attn_weight, float *out,
                         int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                         int64_t L, int64_t K, uint32_t flags, void *stream);

/*
 * Bytes of device workspace msda_backward needs for these sizes (0 when
 * nothing is launched or the sizes are invalid).  It depends on the sizes
 * only, not on the level table: 64 bytes per sampling point (room for one
 * 16-byte record per 8x8 value tile the point's neighbours touch, at most
 * four) plus about 32 bytes per tile bound and head.  This is the size for
 * the fastest call, which sorts every point's records at once.
 */
size_t msda_backward_workspace_size(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                    int64_t L, int64_t K);

/*
 * The smallest workspace msda_backward accepts for these sizes (0 as for
 * msda_backward_workspace_size): the layout of one pass over one head of one
 * batch and min(Nq, 1024) queries.  Given less than
 * msda_backward_workspace_size, the backward computes grad_value in passes,
 * one after another on `stream`, each over a box of batches x heads x
 * queries whose layout fits the workspace, as few as the workspace allows:
 * groups of whole batches; else ranges of queries of one batch with every
 * head (the passes after a range's first adding to grad_value); else, below
 * room for 1024 queries of every head, groups of heads and ranges of
 * queries.  The gradients are the same up to summation order; each pass
 * costs its own launches (at the encoder shape about 60 us: 345 us in one
 * pass, 716 us in the 6 passes of 64 MiB).
 */
size_t msda_backward_workspace_min(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                   int64_t L, int64_t K);

/*
 * Backward of msda_forward for the upstream gradient grad_out.  The pages give
 * no formulas (first page, section 2.3 says the interpolation is differentiable
 * so the gradient reaches the offsets); these are the exact derivatives of the
 * forward above.  With the four neighbours' bilinear weights w_c, values v_c
 * (zero outside the map) and fractional parts fx, fy of the pixel coordinate:
 *   grad_attn_weight = sum_d g_d * sum_c w_c v_c,d
 *   grad_loc.x = A * W_l * sum_d g_d * ((1-fy)(v_TR - v_TL) + fy (v_BR - v_BL))_d
 *   grad_loc.y = A * H_l * sum_d g_d * ((1-fx)(v_BL - v_TL) + fx (v_BR - v_TR))_d
 *   grad_value[neighbour c] += A * w_c * g             (summed over all points)
 * At an integer pixel coordinate the derivative is the one of the cell
 * [x0, x0+1) chosen by the floor.
 *
 * workspace: a DEVICE buffer of at least msda_backward_workspace_min(...)
 * bytes (msda_backward_workspace_size(...) for a single pass), 256-byte
 * aligned, owned by the caller; its contents on entry do not matter and are
 * clobbered; workspace_bytes is its size.  Calls that overlap in time (other streams) need
 * separate workspaces.
 *
 * flags: MSDA_BWD_ACCUMULATE and/or MSDA_ALIGN_CORNERS (the latter as given to
 * the forward), MSDA_BWD_BINNED.  grad_value is overwritten unless flags has
 * MSDA_BWD_ACCUMULATE, in which case the gradient is added to it.  Its
 * summation order is not fixed, so repeated calls may differ in the last
 * bits.  grad_sampling_loc and grad_attn_weight are overwritten and
 * deterministic.  With a level table msda_validate_host rejects, the
 * gradients are unspecified (memory outside the tensors is still never
 * touched).
 *
 * stream, side_stream, side_events: see "Streams and errors" above.
 *
 * Heads of at most 256 points (Nq * L * K <= 256 per (batch, head)) run as
 * one kernel on `stream`, a workgroup per (batch, head, 256 pixels); all
 * others, and every call with MSDA_BWD_BINNED, run the binned pipeline.  Both
 * compute the same gradients; the workspace is required either way.
 */
msda_status msda_backward(const void *value, int value_dtype,
                          const int64_t *spatial_shapes, const int64_t *level_start_index,
                          const float *sampling_loc, const float *attn_weight,
                          const float *grad_out, float *grad_value,
                          float *grad_sampling_loc, float *grad_attn_weight,
                          int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                          int64_t L, int64_t K, void *workspace, size_t workspace_bytes,
                          uint32_t flags, void *stream, void *side_stream,
                          void *const *side_events);

/*
 * msda_backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, stream behaviour
 * and results as msda_backward, with the workspace taken from a static
 * device array of MSDA_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * each GPU it runs on until the process ends.  The call allocates nothing
 * (the array's address is looked up once per device, on the first call with
 * that device current).  Problems whose msda_backward_workspace_size exceeds
 * MSDA_NOALLOC_SCRATCH_BYTES run in passes (see msda_backward_workspace_min);
 * those whose msda_backward_workspace_min exceeds it are rejected with
 * MSDA_ERR_SCRATCH before any work is enqueued.  Every call on one GPU uses
 * the same array, and each call clears what it needs: calls that overlap in
 * time on one GPU (other streams, other threads) race on it and must not be
 * made.
 */
#define MSDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
msda_status msda_backward_noalloc(const void *value, int value_dtype,
                                  const int64_t *spatial_shapes, const int64_t *level_start_index,
                                  const float *sampling_loc, const float *attn_weight,
                                  const float *grad_out, float *grad_value,
                                  float *grad_sampling_loc, float *grad_attn_weight,
                                  int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                  int64_t L, int64_t K, uint32_t flags, void *stream,
                                  void *side_stream, void *const *side_events);

/*
 * Measurement entry point: msda_backward with the same arguments and the same
 * work on the same streams, which in addition records caller-owned HIP events
 * around each of its MSDA_BWD_STAGES stages: events[2i] just before the
 * stage's kernel and events[2i + 1] just after it, on the stream that runs it
 * (stage 0 runs on side_stream when the call uses one, the others on
 * `stream`).
 * Nothing is synchronized; once the caller has waited for `stream`,
 * hipEventElapsedTime(events[2i], events[2i + 1]) is the duration of stage i.
 * Stages:
 *   0 grad_attn_weight / grad_sampling_loc   1 workspace clear
 *   2 points per value tile   3 count scan (work list; in overwrite mode the
 *   list of tiles to zero)   4 zeroing of the listed tiles, then the record
 *   scatter into tiles   5 grad_value tiles
 * A small problem (see msda_backward) runs as one kernel, recorded as stage 0;
 * its other stages are empty.  Without a side stream, the stage-0 kernel
 * also clears the bin counters, so stage 1 then holds only grad_value's
 * zero-fill (when there is one).  With grad_value in several passes (a
 * workspace below msda_backward_workspace_size), stages 1-5 are recorded
 * from their start in the first pass to their end in the last.
 * events: 2 * MSDA_BWD_STAGES hipEvent_t created by the caller (with timing);
 * a null entry is skipped (an event record costs the stream a few
 * microseconds, so a caller timing one stage passes only its two events).
 * events itself must not be NULL (MSDA_ERR_NULL).  The library keeps no
 * reference to them.
 */
#define MSDA_BWD_STAGES 6
msda_status msda_backward_events(const void *value, int value_dtype,
                                 const int64_t *spatial_shapes, const int64_t *level_start_index,
                                 const float *sampling_loc, const float *attn_weight,
                                 const float *grad_out, float *grad_value,
                                 float *grad_sampling_loc, float *grad_attn_weight,
                                 int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                 int64_t L, int64_t K, void *workspace, size_t workspace_bytes,
                                 uint32_t flags, void *stream, void *side_stream,
                                 void *const *side_events, void *const *events);

/*
 * Fused prologue.  The module around the core ("Deformable attention:
 * multi-scale sparse sampling and detection practice", section 3.2; the
 * "Deformable DETR" tutorial's pseudocode, section 6) predicts per point a
 * pixel offset and an attention logit; the location is the query's
 * reference point on that level plus the offset divided by the level's
 * (W_l, H_l), and the weights are a softmax of the logits:
 *
 *   loc[b,q,m,l,k] = reference_points[b,q,l] + sampling_offsets[b,q,m,l,k] / (W_l, H_l)
 *   A[b,q,m,l,k]   = S[b,q,m,l,k] * P[b,q,m,l,k], where P is the softmax of
 *                    attn_logits[b,q,m,:] over its L*K entries, or
 *                    (MSDA_SOFTMAX_PER_LEVEL) over the K entries of level l,
 *                    and S the optional scale attention attn_scale (NULL:
 *                    S = 1): the "Deformable DETR" tutorial's multi-scale
 *                    formula (section 3.3) weights each sampled term by a
 *                    separately predicted scale attention S_qlk times A_qlk
 *
 * The module's code normalizes over all L*K points, the same page's text
 * over the K points of each level (section 2.2); both are offered.  The
 * location is computed in fp32 as one correctly rounded division and one
 * addition per coordinate; the softmax in fp32 with its maximum subtracted,
 * then one fp32 product with S.  These entry points evaluate exactly the
 * core above on those locations and weights, without storing them in the
 * forward (unless asked to).
 *
 * Layouts (dense, row-major, device pointers, caller-owned):
 *   reference_points        [B, Nq, L, 2]        fp32, (x, y) normalized
 *   sampling_offsets        [B, Nq, M, L, K, 2]  fp32, (x, y) in pixels of level l
 *   attn_logits             [B, Nq, M, L*K]      fp32 (level-major: index l*K + k)
 *   attn_scale              [B, Nq, M, L, K]     fp32, optional
 *   grad_sampling_offsets   like sampling_offsets
 *   grad_attn_logits        like attn_logits
 *   grad_attn_scale         like attn_scale
 *   grad_reference_points   like reference_points
 * value, the level table, out, grad_out and grad_value as above.
 *
 * msda_forward_fused: out is overwritten.  flags: MSDA_ALIGN_CORNERS and/or
 * MSDA_SOFTMAX_PER_LEVEL.  Errors and limits as msda_forward.
 * sampling_loc_out [B,Nq,M,L,K,2] and attn_weight_out [B,Nq,M,L,K] (fp32) are
 * optional (both NULL, or both given: else MSDA_ERR_NULL): when given they
 * receive the locations and weights (S * P) the forward formed, for a
 * training step to hand to msda_backward_fused instead of having them
 * recomputed.
 */
msda_status msda_forward_fused(const void *value, int value_dtype,
                               const int64_t *spatial_shapes, const int64_t *level_start_index,
                               const float *reference_points, const float *sampling_offsets,
                               const float *attn_logits, const float *attn_scale, float *out,
                               float *sampling_loc_out, float *attn_weight_out,
                               int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                               int64_t L, int64_t K, uint32_t flags, void *stream);

/*
 * Workspace bytes of msda_backward_fused: msda_backward_workspace_size plus
 * 12 bytes per sampling point (the locations and weights, recomputed) and
 * 8 bytes per (batch, query, head, level).  _min: the same with
 * msda_backward_workspace_min in place of msda_backward_workspace_size (the
 * grad_value pipeline then runs in passes, as for msda_backward).
 */
size_t msda_backward_fused_workspace_size(int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                                          int64_t D, int64_t L, int64_t K);
size_t msda_backward_fused_workspace_min(int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                                         int64_t D, int64_t L, int64_t K);

/*
 * Backward of msda_forward_fused: the chain rule through the prologue on top
 * of the core's gradients (msda_backward):
 *   grad_sampling_offsets = grad_loc / (W_l, H_l)
 *   grad_attn_logits      = P * (S grad_A - sum over the softmax group of P * S grad_A)
 *   grad_attn_scale       = P * grad_A
 *   grad_reference_points[b,q,l] = sum over heads m and points k of grad_loc
 * grad_value is overwritten, or added to with MSDA_BWD_ACCUMULATE; the other
 * gradients are overwritten.  grad_reference_points may be NULL (not
 * computed, e.g. for fixed encoder reference points); attn_scale and
 * grad_attn_scale are both NULL (no scale attention) or both given (else
 * MSDA_ERR_NULL), and attn_scale must be the one given to the forward; every
 * other pointer is required.  flags: MSDA_BWD_ACCUMULATE, MSDA_ALIGN_CORNERS and
 * MSDA_SOFTMAX_PER_LEVEL, the last two as given to the forward.
 * sampling_loc / attn_weight: both NULL (the locations and weights are
 * recomputed from the raw inputs into the workspace), or both the arrays
 * msda_forward_fused stored for these same inputs and flags (then they are
 * read instead; anything else gives the gradients at those locations and
 * weights, not at the raw inputs').
 * workspace: at least msda_backward_fused_workspace_min(...) bytes
 * (msda_backward_fused_workspace_size(...) for one pass), 256-byte aligned,
 * as for msda_backward.
 * events: NULL, or 2 * MSDA_BWD_FUSED_STAGES caller-owned HIP events recorded
 * around the stages as msda_backward_events does (null entries skipped):
 * stages 0-5 as there, 6 the prologue (locations and weights into the
 * workspace; empty when they are passed in), 7 the epilogue (what remains of
 * the logit and reference-point gradients; empty when nothing remains).
 * stream, side_stream, side_events as for msda_backward.
 */
#define MSDA_BWD_FUSED_STAGES (MSDA_BWD_STAGES + 2)
msda_status msda_backward_fused(const void *value, int value_dtype,
                                const int64_t *spatial_shapes, const int64_t *level_start_index,
                                const float *reference_points, const float *sampling_offsets,
                                const float *attn_logits, const float *attn_scale,
                                const float *sampling_loc, const float *attn_weight,
                                const float *grad_out, float *grad_value,
                                float *grad_sampling_offsets, float *grad_attn_logits,
                                float *grad_attn_scale, float *grad_reference_points,
                                int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                int64_t L, int64_t K, void *workspace, size_t workspace_bytes,
                                uint32_t flags, void *stream, void *side_stream,
                                void *const *side_events, void *const *events);

/*
 * 3-D (trilinear) variant.  "Deformable attention: multi-scale sparse
 * sampling and detection practice", section 5.3: for point-cloud detection
 * the points fall on voxel (or BEV) features, the offsets gain a z
 * component and bilinear interpolation becomes trilinear -- the 2-D core with
 * one more coordinate:
 *
 *     out[b, q, m*D + d] = sum_l sum_k A[b,q,m,l,k] * T_l(value[b, :, m, d], loc[b,q,m,l,k])
 *
 * Level l is a Z_l x H_l x W_l volume flattened z-major (voxel (x, y, z) is
 * row start_l + (z*H_l + y)*W_l + x); a location is normalized (u, v, w) along
 * (x, y, z) and maps to the voxel coordinate x = u*W_l - 0.5, y = v*H_l - 0.5,
 * z = w*Z_l - 0.5 (each one fp32 fused multiply-add, then floored), or with
 * MSDA_ALIGN_CORNERS x = u*(W_l - 1) etc.  T_l sums the eight integer
 * neighbours with the product of the three tent weights; neighbours outside
 * the volume contribute zero.
 *
 * Layouts as the 2-D core except
 *   volume_shapes      [L, 3]  int64, rows (Z_l, H_l, W_l)
 *   sampling_loc       [B, Nq, M, L, K, 3]    fp32, last axis (x, y, z) = (u, v, w)
 *   grad_sampling_loc  [B, Nq, M, L, K, 3]
 * with Nv = sum_l Z_l*H_l*W_l.  Limits as the 2-D core, with
 * Nq*M*L*K*3 < 2^31 and each extent < 2^24.
 *
 * msda3d_forward: out is overwritten; flags 0 or MSDA_ALIGN_CORNERS.
 * msda3d_backward: the exact derivatives, as for the 2-D core with the
 * eight neighbours (grad_loc.z carries the factor Z_l, or Z_l - 1 with
 * MSDA_ALIGN_CORNERS).  grad_value is overwritten unless flags has
 * MSDA_BWD_ACCUMULATE; it is summed per 8x8 tile of each plane as in the 2-D
 * backward (the records of a tile arrive in no fixed order; with heads of 64
 * channels or more a tile split over several work items is also added to
 * atomically), so its last bits may differ between calls; grad_sampling_loc and grad_attn_weight are
 * overwritten and deterministic.  workspace: at least
 * msda3d_backward_workspace_min(...) bytes, msda3d_backward_workspace_size(...)
 * for one pass (128 bytes per point -- up to eight 16-byte records, two
 * planes of four tiles -- plus about 16 bytes per voxel and head); with less
 * than the latter grad_value is computed in passes as for msda_backward;
 * 256-byte aligned, caller-owned, contents irrelevant.  stream, side_stream,
 * side_events as for msda_backward; also needs Nq <= 2^25.
 */
size_t msda3d_backward_workspace_size(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                      int64_t L, int64_t K);
size_t msda3d_backward_workspace_min(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                     int64_t L, int64_t K);

msda_status msda3d_forward(const void *value, int value_dtype,
                           const int64_t *volume_shapes, const int64_t *level_start_index,
                           const float *sampling_loc, const float *attn_weight, float *out,
                           int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                           int64_t L, int64_t K, uint32_t flags, void *stream);

msda_status msda3d_backward(const void *value, int value_dtype,
                            const int64_t *volume_shapes, const int64_t *level_start_index,
                            const float *sampling_loc, const float *attn_weight,
                            const float *grad_out, float *grad_value,
                            float *grad_sampling_loc, float *grad_attn_weight,
                            int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                            int64_t L, int64_t K, void *workspace, size_t workspace_bytes,
                            uint32_t flags, void *stream, void *side_stream,
                            void *const *side_events);

/* msda_validate_host for the 3-D variant: a HOST copy of volume_shapes [L, 3]. */
msda_status msda3d_validate_host(const int64_t *volume_shapes_host,
                                 const int64_t *level_start_host,
                                 int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                 int64_t L, int64_t K);

/*
 * DAT sampled-key attention.  DAT (the Deformable Attention Transformer; its
 * DAttentionBaseline walk-through, sections 2.1 to 2.3, and the first page's
 * section 5.1) samples Ns keys/values per offset group at reference points
 * moved by predicted offsets -- msda_forward / msda_backward with L = 1,
 * K = 1, attention weight 1 and MSDA_ALIGN_CORNERS, the grid_sample call of
 * its section 2.2 -- and then runs standard multi-head attention of all N
 * query tokens against them (section 2.3).  These two calls are that
 * attention, per batch b and head h:
 *
 *     S = scale * Q K^T + bias,   P = softmax of S over the Ns keys,   O = P V
 *
 * bias is the deformable relative-position bias, whose construction the page
 * elides: an optional dense input here (NULL = none).  fp32 throughout, the
 * products on the matrix cores (fp32 MFMA), accumulation in fp32.
 *
 * Layouts (dense, row-major, channel-last, device pointers, caller-owned):
 *   q, out, grad_q, grad_out     [B, N, heads, head_dim]   fp32
 *   k, v, grad_k, grad_v         [B, Ns, heads, head_dim]  fp32
 *   bias, grad_bias              [B, heads, N, Ns]         fp32 (optional)
 *   lse                          [B, heads, N]             fp32: log sum_keys exp(S), written
 *                                by the forward, read by the backward
 * Limits: head_dim in {16, 32, 64}; 1 <= Ns <= 256 (<= 240 for head_dim 64:
 * one (b, head)'s keys fit 64 KB of LDS); B*heads < 65536; N*Ns < 2^29.
 * B or N may be 0.
 *
 * msda_dat_attention_forward: out and lse are overwritten.
 * msda_dat_attention_backward: grad_q, grad_k, grad_v and (when grad_bias is
 * not NULL; then bias must not be NULL either, and Ns % 4 == 0 keeps its
 * stores vectorized) grad_bias are overwritten.  grad_k and grad_v may be
 * summed with fp32 atomics over ranges of queries, so their last bits may
 * differ between calls.  workspace: at least
 * msda_dat_attention_workspace_size(...) bytes of device memory (4 bytes per
 * (b, head, query): rowsum(dO * O)), contents irrelevant.
 */
msda_status msda_dat_attention_forward(const float *q, const float *k, const float *v,
                                       const float *bias, float *out, float *lse,
                                       int64_t B, int64_t N, int64_t Ns, int64_t heads,
                                       int64_t head_dim, float scale, void *stream);

size_t msda_dat_attention_workspace_size(int64_t B, int64_t N, int64_t Ns, int64_t heads,
                                         int64_t head_dim);

msda_status msda_dat_attention_backward(const float *q, const float *k, const float *v,
                                        const float *bias, const float *out, const float *lse,
                                        const float *grad_out, float *grad_q, float *grad_k,
                                        float *grad_v, float *grad_bias, void *workspace,
                                        size_t workspace_bytes, int64_t B, int64_t N,
                                        int64_t Ns, int64_t heads, int64_t head_dim,
                                        float scale, void *stream);

/*
 * Pure host check of the sizes and of a HOST copy of the level table:
 * H_l, W_l >= 1, level_start_host[l] = sum of H*W of levels before l,
 * Nv = sum H*W, plus every limit msda_forward/msda_backward check.
 * Needs no GPU.
 */
msda_status msda_validate_host(const int64_t *spatial_shapes_host,
                               const int64_t *level_start_host,
                               int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                               int64_t L, int64_t K);

/* Static English text for a status code (never NULL). */
const char *msda_status_string(int status);

/* hipError_t of the last MSDA_ERR_HIP returned on this thread (0 if none). */
int msda_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_H */

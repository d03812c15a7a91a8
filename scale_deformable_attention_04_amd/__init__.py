"""MI355X-native multi-scale deformable attention (MSDeformAttn) sampling core.

``forward`` / ``backward`` call the C ABI of libmsda.so (include/msda.h): hand
written gfx950 HIP kernels.  ``ms_deform_attn`` wraps them as a
torch.autograd.Function.  torch is used for device memory and the stream only.
"""
from __future__ import annotations

import torch

from ._binding import (BWD_FUSED_STAGES, BWD_STAGES, EXPORTED, LIB_PATH, MSDA_ALIGN_CORNERS,
                       MSDA_BF16, MSDA_BWD_ACCUMULATE, MSDA_ERR_DTYPE,
                       MSDA_ERR_HIP, MSDA_ERR_NULL, MSDA_ERR_SCRATCH, MSDA_ERR_SHAPE,
                       MSDA_ERR_UNSUPPORTED, MSDA_ERR_WORKSPACE, MSDA_F32, MSDA_OK,
                       MSDA_SOFTMAX_PER_LEVEL, MSDAError, NOALLOC_SCRATCH_BYTES,
                       backward, backward3d, backward_fused, backward_noalloc, dat_attention,
                       dat_attention_backward, dat_sample, dat_sample_backward, forward,
                       forward3d, forward_fused, fused_workspace_min, fused_workspace_size,
                       load, make_events, stage_times, status_string, validate_host,
                       validate_host3d, workspace_min, workspace_min3d, workspace_size,
                       workspace_size3d)

__all__ = ["forward", "backward", "backward_noalloc", "NOALLOC_SCRATCH_BYTES",
           "forward_fused", "backward_fused", "BWD_STAGES",
           "BWD_FUSED_STAGES", "make_events", "stage_times", "workspace_size",
           "workspace_min", "fused_workspace_size", "fused_workspace_min", "workspace_size3d",
           "workspace_min3d", "validate_host", "status_string", "load",
           "MSDAError",
           "ms_deform_attn", "MSDeformAttnFunction", "ms_deform_attn_fused",
           "MSDeformAttnFusedFunction", "forward3d", "backward3d", "validate_host3d",
           "ms_deform_attn_3d", "MSDeformAttn3dFunction", "dat_sample", "dat_sample_backward",
           "dat_attention", "dat_attention_backward", "DATSampleFunction",
           "DATAttentionFunction", "dat_deformable_attention", "LIB_PATH", "EXPORTED"]


class MSDeformAttnFunction(torch.autograd.Function):
    """out = core(value, level table, sampling_loc, attn_weight) with the
    library's backward.  grad_value comes back in fp32; autograd casts it to
    value's dtype.  The level table is checked on the host only with
    validate=True (a device-to-host copy); the kernels never touch memory
    outside the tensors whatever it holds."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start_index, sampling_loc, attn_weight,
                align_corners=False, validate=False):
        out = forward(value, spatial_shapes, level_start_index, sampling_loc, attn_weight,
                      align_corners=align_corners, validate=validate)
        ctx.save_for_backward(value, spatial_shapes, level_start_index, sampling_loc,
                              attn_weight)
        ctx.align_corners = align_corners
        return out

    @staticmethod
    def backward(ctx, grad_out):
        value, ss, st, loc, attn = ctx.saved_tensors
        gv, gl, ga = backward(value, ss, st, loc, attn, grad_out.contiguous(), validate=False,
                              align_corners=ctx.align_corners)
        return gv, None, None, gl, ga, None, None


def ms_deform_attn(value, spatial_shapes, level_start_index, sampling_loc, attn_weight,
                   align_corners=False, validate=False):
    return MSDeformAttnFunction.apply(value, spatial_shapes, level_start_index, sampling_loc,
                                      attn_weight, align_corners, validate)


class MSDeformAttnFusedFunction(torch.autograd.Function):
    """out = core(value, level table, ref + offsets / (W_l, H_l), S * softmax(logits))
    computed by the fused entry points (scale S optional); the backward
    returns the gradients of value, reference_points, sampling_offsets,
    attn_logits and scale."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start_index, reference_points,
                sampling_offsets, attn_logits, per_level=False, align_corners=False,
                scale=None, validate=False):
        # with a backward to come, the forward also stores the locations and
        # weights it forms, so the backward does not recompute them
        save = any(ctx.needs_input_grad)
        res = forward_fused(value, spatial_shapes, level_start_index, reference_points,
                            sampling_offsets, attn_logits, per_level=per_level,
                            align_corners=align_corners, save=save, scale=scale,
                            validate=validate)
        out, loc, attn = res if save else (res, None, None)
        ctx.save_for_backward(value, spatial_shapes, level_start_index, reference_points,
                              sampling_offsets, attn_logits, loc, attn, scale)
        ctx.per_level = per_level
        ctx.align_corners = align_corners
        return out

    @staticmethod
    def backward(ctx, grad_out):
        value, ss, st, ref, off, logits, loc, attn, scale = ctx.saved_tensors
        res = backward_fused(value, ss, st, ref, off, logits, grad_out.contiguous(),
                             validate=False, need_grad_ref=ctx.needs_input_grad[3],
                             per_level=ctx.per_level, align_corners=ctx.align_corners,
                             saved=None if loc is None else (loc, attn), scale=scale)
        gv, goff, gz, gref = res[:4]
        gs = res[4] if scale is not None else None
        return gv, None, None, gref, goff, gz, None, None, gs, None


def ms_deform_attn_fused(value, spatial_shapes, level_start_index, reference_points,
                         sampling_offsets, attn_logits, per_level=False, align_corners=False,
                         scale=None, validate=False):
    return MSDeformAttnFusedFunction.apply(value, spatial_shapes, level_start_index,
                                           reference_points, sampling_offsets, attn_logits,
                                           per_level, align_corners, scale, validate)


class MSDeformAttn3dFunction(torch.autograd.Function):
    """The 3-D (trilinear) core with the library's backward (validate as for
    MSDeformAttnFunction)."""

    @staticmethod
    def forward(ctx, value, volume_shapes, level_start_index, sampling_loc, attn_weight,
                align_corners=False, validate=False):
        out = forward3d(value, volume_shapes, level_start_index, sampling_loc, attn_weight,
                        align_corners=align_corners, validate=validate)
        ctx.save_for_backward(value, volume_shapes, level_start_index, sampling_loc, attn_weight)
        ctx.align_corners = align_corners
        return out

    @staticmethod
    def backward(ctx, grad_out):
        value, ss, st, loc, attn = ctx.saved_tensors
        gv, gl, ga = backward3d(value, ss, st, loc, attn, grad_out.contiguous(), validate=False,
                                align_corners=ctx.align_corners)
        return gv, None, None, gl, ga, None, None


def ms_deform_attn_3d(value, volume_shapes, level_start_index, sampling_loc, attn_weight,
                      align_corners=False, validate=False):
    return MSDeformAttn3dFunction.apply(value, volume_shapes, level_start_index, sampling_loc,
                                        attn_weight, align_corners, validate)


class DATSampleFunction(torch.autograd.Function):
    """DAT's deformable sampling: features [B, H*W, G, Dg] at positions
    [B, Ns, G, 2] -> [B, Ns, G*Dg], with gradients for both."""

    @staticmethod
    def forward(ctx, x, hw, pos):
        ctx.save_for_backward(x, pos)
        ctx.hw = tuple(int(v) for v in hw)
        return dat_sample(x, ctx.hw, pos, validate=False)

    @staticmethod
    def backward(ctx, grad):
        x, pos = ctx.saved_tensors
        gx, gp = dat_sample_backward(x, ctx.hw, pos, grad, validate=False)
        return gx, None, gp


class DATAttentionFunction(torch.autograd.Function):
    """softmax(scale * Q K^T + bias) V per (batch, head) on the matrix cores."""

    @staticmethod
    def forward(ctx, q, k, v, bias=None, scale=None):
        out, lse = dat_attention(q, k, v, bias, scale)
        ctx.save_for_backward(q, k, v, bias, out, lse)
        ctx.scale = scale
        return out

    @staticmethod
    def backward(ctx, grad_out):
        q, k, v, bias, out, lse = ctx.saved_tensors
        need_b = bias is not None and ctx.needs_input_grad[3]
        gq, gk, gv, gb = dat_attention_backward(q, k, v, out, lse, grad_out.contiguous(), bias,
                                                need_grad_bias=need_b, scale=ctx.scale)
        return gq, gk, gv, gb, None


def dat_deformable_attention(q, k, v, bias=None, scale=None):
    return DATAttentionFunction.apply(q, k, v, bias, scale)

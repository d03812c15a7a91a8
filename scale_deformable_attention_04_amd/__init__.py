"""MI355X-native multi-scale deformable attention (MSDeformAttn) sampling core.

``forward`` / ``backward`` call the C ABI of libmsda.so (include/msda.h): hand
written gfx950 HIP kernels.  ``ms_deform_attn`` wraps them as a
torch.autograd.Function.  torch is used for device memory and the stream only.
"""
from __future__ import annotations

import torch

from ._binding import (BWD_STAGES, EXPORTED, LIB_PATH, MSDA_ALIGN_CORNERS, MSDA_BF16,
                       MSDA_BWD_ACCUMULATE, MSDA_ERR_DTYPE,
                       MSDA_ERR_HIP, MSDA_ERR_NULL, MSDA_ERR_SHAPE, MSDA_ERR_UNSUPPORTED,
                       MSDA_ERR_WORKSPACE, MSDA_F32, MSDA_OK, MSDAError, backward, forward, load,
                       make_events, stage_times, status_string, validate_host, workspace_size)

__all__ = ["forward", "backward", "BWD_STAGES", "make_events", "stage_times", "workspace_size",
           "validate_host", "status_string", "load",
           "MSDAError",
           "ms_deform_attn", "MSDeformAttnFunction", "LIB_PATH", "EXPORTED"]


class MSDeformAttnFunction(torch.autograd.Function):
    """out = core(value, level table, sampling_loc, attn_weight) with the
    library's backward.  grad_value comes back in fp32; autograd casts it to
    value's dtype."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start_index, sampling_loc, attn_weight,
                align_corners=False):
        out = forward(value, spatial_shapes, level_start_index, sampling_loc, attn_weight,
                      align_corners=align_corners)
        ctx.save_for_backward(value, spatial_shapes, level_start_index, sampling_loc,
                              attn_weight)
        ctx.align_corners = align_corners
        return out

    @staticmethod
    def backward(ctx, grad_out):
        value, ss, st, loc, attn = ctx.saved_tensors
        gv, gl, ga = backward(value, ss, st, loc, attn, grad_out.contiguous(), validate=False,
                              align_corners=ctx.align_corners)
        return gv, None, None, gl, ga, None


def ms_deform_attn(value, spatial_shapes, level_start_index, sampling_loc, attn_weight,
                   align_corners=False):
    return MSDeformAttnFunction.apply(value, spatial_shapes, level_start_index, sampling_loc,
                                      attn_weight, align_corners)

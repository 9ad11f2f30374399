"""Parallax (parameterized Local Linear Attention) forward and backward on AMD MI355X,
with the kernels around it: fused input projections, a Walsh-Hadamard output
projection and Based linear attention.

The compute path is the gfx950 HIP library ``libparallax.so`` (C ABI in
``include/parallax.h``); this package only builds it and marshals torch
tensors into it.
"""
from .binding import (EXPORTED, LIBRARY, ParallaxError, based_state_shape, load_library,
                      parallax_attn_bwd, parallax_based_decode, parallax_based_fwd,
                      parallax_based_state_floats, parallax_based_workspace_size,
                      parallax_attn_bwd_workspace_size, parallax_attn_decode,
                      parallax_attn_decode_paged, parallax_attn_decode_paged_workspace_size,
                      parallax_attn_fwd, parallax_attn_fwd_f32,
                      parallax_attn_fwd_noalloc, parallax_attn_fwd_precise,
                      parallax_attn_fwd_train, parallax_attn_fwd_workspace_size,
                      parallax_hadamard_out, parallax_qkvr_project, parallax_status_string,
                      split_qkvr)

__all__ = ["EXPORTED", "LIBRARY", "ParallaxError", "based_state_shape", "load_library",
           "parallax_attn_bwd", "parallax_based_decode", "parallax_based_fwd",
           "parallax_based_state_floats", "parallax_based_workspace_size",
           "parallax_attn_bwd_workspace_size", "parallax_attn_decode",
           "parallax_attn_decode_paged", "parallax_attn_decode_paged_workspace_size",
           "parallax_attn_fwd", "parallax_attn_fwd_f32",
           "parallax_attn_fwd_noalloc",
           "parallax_attn_fwd_precise",
           "parallax_attn_fwd_train", "parallax_attn_fwd_workspace_size",
           "parallax_hadamard_out", "parallax_qkvr_project", "parallax_status_string", "split_qkvr"]

"""Joint video-audio attention hot path for MI355X (gfx950).

A C-ABI library (libmmdit.so, include/mmdit.h) of hand-written HIP kernels:
time-shifted 3D RoPE, joint self-attention (forward, forward with the
log-sum-exp, and backward), bidirectional audio<->video cross-attention and
Prism-style block-sparse video self-attention with uniform or content-adaptive
block shapes.  This
package is its thin Python binding; importing it does not load the library,
the first call does (and raises if the library was not built).
"""
from ._lib import (  # noqa: F401
    MmditError, RopeSpec, layout_segments, lib, mmdit_abi_version, mmdit_av_cross_attn,
    mmdit_adaptive_tile_table, mmdit_block_sparse_attn, mmdit_block_sparse_attn_adaptive,
    mmdit_block_sparse_attn_adaptive_bwd,
    mmdit_block_sparse_attn_bwd,
    mmdit_block_sparse_attn_fwd, mmdit_joint_attn, mmdit_joint_attn_bwd, mmdit_joint_attn_fwd, mmdit_last_error,
    mmdit_joint_attn_noalloc, MMDIT_NOALLOC_SCRATCH_BYTES, mmdit_joint_attn_rope, MMDIT_OP_JOINT_ATTN_ROPE,
    mmdit_rope3d, mmdit_rope3d_build_table, mmdit_rope3d_table_floats, mmdit_token_norms, mmdit_workspace_bytes,
    sparse_desc, ADAPTIVE_SHAPES,
    MMDIT_OP_JOINT_ATTN, MMDIT_OP_AV_CROSS_ATTN, MMDIT_OP_BLOCK_SPARSE_ATTN, MMDIT_OP_JOINT_ATTN_BWD,
    MMDIT_OP_BLOCK_SPARSE_ATTN_BWD, MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE, MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE_BWD,
    MMDIT_FP32,
    MMDIT_BF16,
)


def rope_spec_for(w):
    """RoPE descriptor of a workload dict (T, H, W, n_cond_frames, n_audio,
    n_text, heads, head_dim, split, theta, audio_scale)."""
    segs, n = layout_segments(w["T"], w["H"], w["W"], w.get("n_cond_frames", 0),
                              w.get("n_audio", 0), w.get("n_text", 0), w.get("audio_scale"))
    return RopeSpec(segs, n, w["heads"], w["head_dim"], w["split"], w.get("theta", 10000.0))

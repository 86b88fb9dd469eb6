"""segment_causal_attention_amd: Python binding of libnomas, segment-causal
attention over a lifelong INT8 KV cache for AMD MI355X (gfx950).

The compute path is the HIP library libnomas.so (C ABI: include/nomas.h);
this package only marshals arguments.  Build it with
``python -m segment_causal_attention_amd.build`` (or __graft_entry__.build()).
"""
from ._lib import (  # noqa: F401
    EHIP, ECAPACITY, EINVAL, EUNSUPPORTED, HEAD_DIM, MAX_CAM, MAX_SEGS, MAX_SEL_RANGES, MAX_SPLIT, OK, SM_SCALE,
    SYMBOLS,
    W8A16_NOALLOC_MAX_BYTES, NomasError, Seg, cam_tokens, cam_xattn, cam_xattn_workspace, gqa_attn, gqa_attn_workspace, kv_quant_append, lib, rope3d, rope_table, seg_array,
    seg_attn, seg_attn_bwd, seg_attn_bwd_workspace, seg_attn_workspace, seg_tokens, sel_arrays, shutdown, strerror, version, w8a16_linear, w8a16_linear_noalloc, w8a16_linear_workspace,
)

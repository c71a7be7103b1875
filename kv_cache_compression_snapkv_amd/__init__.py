"""AnchorKV anchor-residual KV-cache hot path on AMD MI355X (gfx950).

compress: end-of-prefill compression of K/V into anchors + (index, gamma)
pointers + 2-bit residual records; decode_attn: attention over the compressed
cache without reconstructing it; decode_attn_tail: the same plus an exact tail
of tokens appended after compression.  Both run in hand-written HIP kernels behind
the C ABI in include/anchorkv.h; this package only marshals arguments.
"""
from .binding import (ANCHORS_COVER, ANCHORS_UNIFORM, BF16, CODEC_AFFINE, CODEC_HADAMARD_LM, F32, AnchorKVError, Params, PlanInfo, alloc, cache_layout, compress, decode_attn,
                      decode_attn_noalloc, decode_attn_tail, decode_workspace_bytes, lib, pack_unit, params, plan, plan_from_header,
                      profile_enable, profile_read, unpack_unit, version, workspace_offsets)

__all__ = ["ANCHORS_COVER", "ANCHORS_UNIFORM", "BF16", "CODEC_AFFINE", "CODEC_HADAMARD_LM", "F32", "AnchorKVError", "Params", "PlanInfo", "alloc", "cache_layout", "compress", "decode_attn",
           "decode_attn_noalloc", "decode_attn_tail", "decode_workspace_bytes", "lib", "pack_unit", "params", "plan", "plan_from_header",
           "profile_enable", "profile_read", "unpack_unit", "version", "workspace_offsets"]

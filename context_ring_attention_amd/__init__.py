"""MI355X-native context-parallel ring attention: one CP rank's exact GQA attention on gfx950.

The computation lives in ``libcpattn.so`` (hand-written HIP kernels behind the C ABI of
``include/cpattn.h``); :mod:`context_ring_attention_amd.binding` marshals torch tensors into it.
"""
from .binding import (CP_BF16, CP_F32, CpError, CpSegment, decode_splitkv, decode_workspace,
                      decode_workspace_bytes,
                      last_error, load, merge_lse, partial_attn, ring_pass_kv, ring_pass_q,
                      segments, select_ring_variant, shard_map)

__all__ = ["CP_BF16", "CP_F32", "CpError", "CpSegment", "decode_splitkv", "decode_workspace",
           "decode_workspace_bytes",
           "last_error", "load", "merge_lse", "partial_attn", "ring_pass_kv", "ring_pass_q",
           "segments", "select_ring_variant", "shard_map"]

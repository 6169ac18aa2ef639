"""Engram n-gram embedding hot path on MI355X (gfx950): hash -> row gather -> gradient scatter-add.

The compute lives in ``libengram.so`` (hand-written HIP kernels behind the C ABI
of ``include/engram.h``); this package is its Python binding.
"""
from .engram import (  # noqa: F401
    ENGRAM_BF16, ENGRAM_F32, EngramError, EngramHashSpec, LIB_PATH,
    QWEN3_8_FLASH_NEXT_EMBEDDING_DIM, QWEN3_8_FLASH_NEXT_EOS_TOKEN_ID, QWEN3_8_FLASH_NEXT_LAYER_MULTIPLIERS,
    QWEN3_8_FLASH_NEXT_NGRAM_HEAD_OFFSETS, QWEN3_8_FLASH_NEXT_NGRAM_HEAD_VOCAB_SIZES,
    QWEN3_8_FLASH_NEXT_NGRAM_PADDED_ROWS, engram_gather, engram_hash, engram_hash_gather, engram_hash_gather_slice, engram_hash_slice, engram_scatter_add,
    engram_scatter_add_apply, engram_scatter_add_noalloc, engram_scatter_add_plan, engram_scatter_add_plan_from_tokens, engram_scatter_add_plan_from_tokens_slice, engram_scatter_add_plan_padded, engram_scatter_add_workspace,
    engram_route_plan, engram_route_validate, engram_pack_fixed_capacity, engram_unpack_fixed_capacity,
    engram_permute_rows, engram_unpermute_rows, engram_unpack_unpermute_rows, engram_permute_pack_rows, engram_gather_padded, engram_short_conv, engram_short_conv_backward,
    engram_grouped_rms_norm, engram_grouped_rms_norm_backward, load_library, make_hash_spec, qwen3_8_flash_next_spec,
)

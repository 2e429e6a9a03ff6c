"""lgm: paged GQA/MQA single-token decode attention for AMD MI355X (gfx950).

The compute path is the C-ABI library liblgm.so (include/*.h), built from
the HIP sources in csrc/ by ``python -m paged_gqa_decode_lgm_amd.build``.
This package only marshals arguments to it; nothing here computes any part of
the decode path, and calls fail loudly when the library is missing.
"""
from ._binding import (  # noqa: F401
    LGM_BF16, LGM_CACHE_HND, LGM_ERR_HIP, LGM_ERR_INVALID_ARGUMENT, LGM_ERR_UNSUPPORTED, LGM_ERR_WORKSPACE_TOO_SMALL,
    LGM_F32, LGM_FP4_E2M1, LGM_FP8_E4M3, LGM_OK, LGM_ROPE_INTERLEAVED, LGM_SCALE_PER_TENSOR, LIB_PATH, LgmError, header_functions, lgm_abi_version, lgm_last_error,
    lgm_check_block_tables, lgm_lse_merge, lgm_paged_decode_attn, lgm_paged_decode_attn_static, lgm_paged_decode_partition_size,
    lgm_paged_decode_workspace_size,
    lgm_mla_dims, lgm_paged_dims, lgm_paged_mla_decode, lgm_paged_mla_partition_size, lgm_paged_mla_workspace_size,
    lgm_rope_kv_append, lgm_stream_read_probe, lib, make_dims, make_mla_dims,
)
from . import ops  # noqa: F401

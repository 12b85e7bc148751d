"""MapFlow attention-map compression and fused head-mapped retrieval for MI355X.

The compute lives in libmapflow.so (HIP kernels for gfx950, C boundary in
include/mapflow.h); :mod:`cross_model_sparse_amd.mapflow` is its thin Python
binding over torch device tensors.
"""
from .mapflow import (  # noqa: F401
    MapflowError, CapacityError, abi_version, block_mass, block_mass_ws_bytes, topp_select_bsr,
    topp_select_bsr_noalloc,
    retrieve_fused, retrieve_fused_multi, retrieve_fused_varlen, retrieve_kernel, compress, topp_workspace_bytes, retrieve_workspace_bytes, retrieve_split_workspace_bytes, load, lib_path, EXPORTED,
    row_lse, block_mass_qk, block_mass_qk_workspace_bytes, lse_block_mass_qk,
    lse_block_mass_qk_workspace_bytes, topp_select_bsr_qk, compress_qk,
    BlockManager, prefix_hashes, pool_store,
    MF_OK, MF_ERR_INVALID, MF_ERR_UNSUPPORTED, MF_ERR_CAPACITY, MF_ERR_HIP,
    MF_F32, MF_F16, MF_BF16,
)

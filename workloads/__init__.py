"""Seeded synthetic inputs for paged-KV attention.

This package only draws random numbers and lays them out as a paged KV cache
(page pool, CSR page table, queries). It holds none of the attention
arithmetic: both the fp64 oracle and the GPU path consume the same stored
bytes that it produces.
"""
from .gen import (  # noqa: F401
    Workload,
    make_config,
    config_lengths,
    make_workload,
    make_cascade,
    make_ragged,
    make_block_sparse,
    BlockSparseWorkload,
    RaggedWorkload,
    csr_from_page_lists,
    to_storage_bits,
    to_e4m3_codes,
    CONFIG_NAMES,
    FP8_K_SCALE,
    FP8_V_SCALE,
)

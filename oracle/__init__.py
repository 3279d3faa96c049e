"""CPU oracle of the DSA sparse-attention step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``lightning_indexer_top_02_amd``) and neither imports the
other.  The arithmetic lives in ``dsa_oracle.c`` (plain C, fp64); this package
only builds it, loads it and marshals numpy arrays.
"""
from .oracle import (  # noqa: F401
    build,
    decode_bf16,
    decode_e4m3,
    decode_e8m0,
    encode_e4m3,
    encode_bf16,
    cache_append,
    latent_append,
    visible,
    scores,
    select,
    indexer_topk,
    sparse_attn,
    lib_path,
    load_library,
    restore_library,
)

"""Host logic of bench.py (no GPU): the algorithmic byte and flop counts the
roofline divides by, checked against hand counts on tiny cases."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402
from lightning_indexer_top_02_amd import inputs  # noqa: E402


def _case(idx_dtype, sfa_dtype, D=64):
    return inputs.make_case(name="acct", seed=1, ctx_lens=[100], n_q=1, idx_dtype=idx_dtype, n_heads_idx=4,
                            head_dim_idx=D, topk=16, sfa_dtype=sfa_dtype, n_heads_sfa=16)


def test_algorithmic_bytes_bf16():
    ab = bench.algorithmic_bytes(_case("bf16", "bf16"))
    # keys 100 x 64 x 2, q 4 x 64 x 2, w 4 x 4, 2 block-table entries, 16 indices
    assert ab["indexer"] == 12800 + 512 + 16 + 8 + 64
    # indices, 16 latent rows of 1152 bytes, q (576) and out (512) for 16 heads in bf16
    assert ab["sparse_attn"] == 64 + 16 * 1152 + 16 * (576 + 512) * 2
    assert ab["indexer_flops"] == 2 * 100 * 4 * 64
    assert ab["sparse_attn_flops"] == 2 * 16 * 16 * (576 + 512)


def test_algorithmic_bytes_quantized_routes():
    # fp8 keys: 64 codes + a 4-byte scale per key; q scales 4 bytes per head
    assert bench.algorithmic_bytes(_case("fp8", "bf16"))["indexer"] == 100 * 68 + 4 * 64 + 4 * 8 + 8 + 64
    # MXFP8 keys: 128 codes + 4 E8M0 bytes per key and per q head
    assert bench.algorithmic_bytes(_case("mxfp8", "bf16", D=128))["indexer"] == \
        100 * 132 + 4 * 128 + 4 * (4 + 4) + 8 + 64
    # fp8 latent rows: 656 bytes each; q and out stay bf16
    assert bench.algorithmic_bytes(_case("bf16", "fp8"))["sparse_attn"] == 64 + 16 * 656 + 16 * (576 + 512) * 2


def test_replicas_cover_three_infinity_caches():
    """The 32K decode state (indexer keys and latent rows, ~46 MB) is rotated
    over at least 16 replicas, so the rotated state exceeds the 256 MB
    Infinity Cache three times over; a state above 768 MB needs no replica."""
    c = inputs.decode_32k(sfa_dtype="bf16")
    state = sum(x.numel() * x.element_size() for x in (c.k_cache, c.kv_cache) if x is not None)
    R = bench.replicas_for(c)
    assert R >= 16 and R * state >= 768e6
    big = inputs.make_case(name="big", seed=2, ctx_lens=[262144] * 3, n_q=1, idx_dtype="bf16", n_heads_idx=4,
                           head_dim_idx=64, topk=16, sfa_dtype="bf16", n_heads_sfa=16)
    assert bench.replicas_for(big) == 1


def test_grid_names_every_scope_workload():
    """The grid carries the 32K batch sweep and the batched fp8 (both widths),
    speculative-verify and chunked-prefill workloads."""
    assert {"decode_32k_b8", "decode_32k_b32", "decode_32k_b64", "decode_32k_b128", "batched_fp8_narrow",
            "batched_fp8_wide", "spec_verify", "chunked_prefill"} <= set(bench.GRID)

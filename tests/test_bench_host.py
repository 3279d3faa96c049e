"""Host logic of bench.py (no GPU): the algorithmic byte and flop counts the
roofline divides by, checked against hand counts on tiny cases."""
import json
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
    assert {"decode_32k_b2", "decode_32k_b4", "decode_32k_b8", "decode_32k_b32", "decode_32k_b64", "decode_32k_b128",
            "batched_fp8_narrow",
            "batched_fp8_wide", "spec_verify", "chunked_prefill"} <= set(bench.GRID)


def test_traffic_summary_sums_the_kernels_of_a_call(tmp_path):
    """Per-call HBM bytes: the median per dispatch of each kernel of the stage,
    summed, scaled by the copy factors; other kernels are left out."""
    rows = {
        "FETCH_SIZE": [("void dsa::sfa_bf16<1, false>(dsa::SfaParams)", [100.0, 300.0, 200.0]),
                       ("void dsa::sfa_combine<true, 4>(dsa::SfaParams)", [50.0, 50.0]),
                       ("void dsa::li_fused<1, 128, 0>(dsa::FusedParams)", [10.0]),
                       ("void at::native::copy_kernel(int)", [9999.0])],
        "WRITE_SIZE": [("void dsa::sfa_bf16<1, false>(dsa::SfaParams)", [8.0, 8.0, 8.0]),
                       ("void dsa::sfa_combine<true, 4>(dsa::SfaParams)", [1.0, 3.0]),
                       ("void dsa::li_fused<1, 128, 0>(dsa::FusedParams)", [2.0]),
                       ("void at::native::copy_kernel(int)", [9999.0])],
    }
    paths = {}
    for ctr, kernels in rows.items():
        p = tmp_path / f"{ctr}.csv"
        with open(p, "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for name, vals in kernels:
                for i, v in enumerate(vals):
                    f.write(f'{i},"{name}",{ctr},{v}\n')
        paths[ctr] = str(p)
    out = bench.traffic_summary("w", paths["FETCH_SIZE"], paths["WRITE_SIZE"], "--no-cpu", str(tmp_path))
    sfa = json.load(open(tmp_path / "traffic_sparse_attn_w.json"))
    want = ((200.0 + 50.0) * bench.FETCH_SCALE + (8.0 + 2.0) * bench.WRITE_SCALE) * 1024
    assert abs(sfa["bytes_per_launch"] - want) < 1e-6
    assert sfa["source_hash"] == bench.kernel_source_hash()
    idx = json.load(open(tmp_path / "traffic_indexer_topk_w.json"))
    assert abs(idx["bytes_per_launch"] - (10.0 * bench.FETCH_SCALE + 2.0) * 1024) < 1e-6
    assert not (tmp_path / "traffic_indexer_scores_w.json").exists()
    assert "copy_kernel" not in out and "--pmc FETCH_SIZE" in out

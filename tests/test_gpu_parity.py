"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (see parity.py): Top-K sets bit-exact in exact mode, else equal up to
the 1e-3 threshold band; outputs within 2e-2 (bf16/fp32 storage) of the
oracle run on the GPU's own indices; the fused call equals the two separate
calls bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import parity
from lightning_indexer_top_02_amd import inputs

pytestmark = pytest.mark.gpu


def _run(case, **kw):
    print(f"\n[case] {case.name} seed={case.seed} lens={case.ctx_lens.tolist()[:8]} "
          f"T={case.num_tokens} K={case.topk}", flush=True)
    case = parity.to_device(case)
    stats = parity.check_case(case, **kw)
    print(f"[ok] {case.name}: {stats}", flush=True)
    return case, stats


# --- tiny decode (fp32 indexer 4 x 64, fp32 SFA 16 heads, L = 4096, K = 256) --
@pytest.mark.parametrize("exact", [True, False], ids=["exact", "float"])
def test_tiny_decode(exact):
    _run(inputs.tiny_decode(exact=exact))


def test_tiny_decode_page_permutation_is_bit_identical():
    base = parity.to_device(inputs.tiny_decode())
    perm = parity.to_device(inputs.permute_pages(inputs.tiny_decode(), seed=5))
    i1, o1, l1 = parity.gpu_fused_decode(base)
    i2, o2, l2 = parity.gpu_fused_decode(perm)
    assert torch.equal(i1, i2) and torch.equal(o1, o2) and torch.equal(l1, l2)


def test_repeat_runs_are_bit_identical():
    case = parity.to_device(inputs.decode_32k(ctx_lens=[9000]))
    a = parity.gpu_fused_decode(case)
    b = parity.gpu_fused_decode(case)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# --- 32K decode (bf16 64 x 128, 128 SFA heads, K = 2048) ----------------------
@pytest.mark.parametrize("exact", [True, False], ids=["exact", "float"])
def test_decode_32k(exact):
    _run(inputs.decode_32k(exact=exact))


# --- ragged lengths, several query tokens per request, K above some lengths ----
RAGGED = [1, 63, 64, 65, 300, 4097, 257]
RAGGED_NQ = [1, 1, 2, 4, 3, 1, 4]


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("exact", [True, False], ids=["exact", "float"])
def test_ragged_wide(dtype, exact):
    _run(inputs.make_case(name=f"ragged_wide_{dtype}", seed=77, ctx_lens=RAGGED, n_q=RAGGED_NQ,
                          idx_dtype=dtype, n_heads_idx=64, head_dim_idx=128, topk=256, exact=exact,
                          sfa_dtype="bf16", n_heads_sfa=128))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("exact", [True, False], ids=["exact", "float"])
def test_ragged_narrow(dtype, exact):
    _run(inputs.make_case(name=f"ragged_narrow_{dtype}", seed=78, ctx_lens=RAGGED, n_q=RAGGED_NQ,
                          idx_dtype=dtype, n_heads_idx=4, head_dim_idx=64, topk=100, exact=exact,
                          w_dist="uniform", sfa_dtype="bf16" if dtype != "f32" else "f32",
                          n_heads_sfa=16, sfa_std=1.0))


# fp8 latent cache for the sparse attention (bf16 indexer), every head-tile
# width the kernel picks (16 heads: one tile; 128 heads at one row: one tile
# per workgroup; several rows: four)
@pytest.mark.parametrize("heads", [16, 64, 128])
@pytest.mark.parametrize("exact", [True, False], ids=["exact", "float"])
def test_sfa_fp8_latent(heads, exact):
    _run(inputs.make_case(name=f"kv8_ragged_{heads}h", seed=96, ctx_lens=RAGGED, n_q=RAGGED_NQ, idx_dtype="bf16",
                          n_heads_idx=64, head_dim_idx=128, topk=256, exact=exact, sfa_dtype="fp8",
                          n_heads_sfa=heads))
    _run(inputs.make_case(name=f"kv8_one_row_{heads}h", seed=97, ctx_lens=[5000], n_q=1, idx_dtype="bf16",
                          n_heads_idx=64, head_dim_idx=128, topk=2048, exact=exact, sfa_dtype="fp8",
                          n_heads_sfa=heads))


# head tiles per sparse-attention workgroup by batch (128 heads): 2 and 4
# rows take 2-tile workgroups, 8 rows 4-tile ones
@pytest.mark.parametrize("rows", [2, 4, 8])
@pytest.mark.parametrize("sfa", ["bf16", "fp8"])
def test_sfa_tile_widths_by_batch(rows, sfa):
    _run(inputs.make_case(name=f"tiles_{rows}rows_{sfa}", seed=98 + rows, ctx_lens=[5000 + 777 * r for r in range(rows)],
                          n_q=1, idx_dtype="bf16", n_heads_idx=64, head_dim_idx=128, topk=2048, sfa_dtype=sfa,
                          n_heads_sfa=128))


# fp32 sparse attention: splits of several 16-row chunks (64 single-row
# requests: 4 splits of 64 rows, K = 250 leaves a ragged last chunk), and a
# batch large enough for one split per row (the output written directly)
@pytest.mark.parametrize("heads", [16, 32])
def test_sfa_f32_multi_chunk_splits(heads):
    _run(inputs.make_case(name=f"f32_4splits_{heads}h", seed=83, ctx_lens=[1000 + 7 * r for r in range(64)], n_q=1,
                          idx_dtype="f32", n_heads_idx=4, head_dim_idx=64, topk=250, w_dist="uniform",
                          sfa_dtype="f32", n_heads_sfa=heads, sfa_std=1.0))


def test_sfa_f32_one_split_per_row():
    _run(inputs.make_case(name="f32_1split", seed=84, ctx_lens=[600 + r for r in range(300)], n_q=1,
                          idx_dtype="f32", n_heads_idx=4, head_dim_idx=64, topk=250, w_dist="uniform",
                          sfa_dtype="f32", n_heads_sfa=16, sfa_std=1.0))


@pytest.mark.parametrize("heads", [5, 17, 48])
def test_odd_indexer_head_counts(heads):
    _run(inputs.make_case(name=f"heads{heads}", seed=79, ctx_lens=[5000, 777], n_q=[1, 2],
                          idx_dtype="bf16", n_heads_idx=heads, head_dim_idx=64, topk=512, exact=True,
                          sfa_dtype="bf16", n_heads_sfa=32))


def test_k_equal_and_above_context():
    for K in (640, 641, 700):
        _run(inputs.make_case(name=f"k{K}", seed=80, ctx_lens=[640], n_q=1, idx_dtype="bf16",
                              n_heads_idx=64, head_dim_idx=128, topk=K, sfa_dtype="bf16", n_heads_sfa=64))


# --- batched fp8 route, speculative verify, chunked prefill (reduced sizes) ----
@pytest.mark.parametrize("exact", [True, False], ids=["exact", "float"])
def test_batched_fp8_narrow_small(exact):
    _run(inputs.batched_decode_fp8(batch=8, lo=2000, hi=20000, exact=exact))


@pytest.mark.parametrize("exact", [True, False], ids=["exact", "float"])
def test_spec_verify_small(exact):
    _run(inputs.spec_verify(batch=2, ctx=20000, exact=exact))


@pytest.mark.parametrize("exact", [True, False], ids=["exact", "float"])
def test_chunked_prefill_small(exact):
    _run(inputs.chunked_prefill(prefix=1000, new=300, exact=exact))


# --- many query rows per request: the row-tiled scoring kernel -----------------
# Requests of 300, 17, 130 (a from-scratch prefill: every position is a query
# row) and 5 rows; head counts with and without padding to 16.
PREFILL_LENS = [700, 2000, 130, 64]
PREFILL_NQ = [300, 17, 130, 5]


@pytest.mark.parametrize("dtype,dim,heads", [("bf16", 128, 64), ("bf16", 64, 40), ("fp8", 128, 64),
                                             ("fp8", 64, 23), ("mxfp8", 128, 64), ("mxfp8", 128, 23)])
@pytest.mark.parametrize("exact", [True, False], ids=["exact", "float"])
def test_prefill_ragged_rows(dtype, dim, heads, exact):
    _run(inputs.make_case(name=f"prefill_ragged_{dtype}_{dim}x{heads}", seed=90, ctx_lens=PREFILL_LENS,
                          n_q=PREFILL_NQ, idx_dtype=dtype, n_heads_idx=heads, head_dim_idx=dim, topk=256,
                          sfa_dtype="bf16", n_heads_sfa=16, exact=exact), fused=False)


# A prefill from scratch (every position a query row: the most uneven causal
# work per row block) next to a short chunked request, every row checked.
@pytest.mark.parametrize("exact", [True, False], ids=["exact", "float"])
def test_scratch_prefill_rows(exact):
    _run(inputs.make_case(name="scratch_prefill_1203", seed=95, ctx_lens=[1203, 500], n_q=[1203, 37],
                          idx_dtype="bf16", n_heads_idx=64, head_dim_idx=128, topk=256, sfa_dtype="bf16",
                          n_heads_sfa=16, exact=exact), fused=False)


# --- scores alone (dsa_indexer_scores) against the oracle's scores -------------
SCORE_CASES = {
    "tiny_f32": lambda exact: inputs.tiny_decode(exact=exact),
    "ragged_bf16": lambda exact: inputs.make_case(name="sc_bf16", seed=91, ctx_lens=PREFILL_LENS, n_q=PREFILL_NQ,
                                                  idx_dtype="bf16", n_heads_idx=64, head_dim_idx=128, topk=64,
                                                  sfa_dtype=None, exact=exact),
    "ragged_fp8_d64": lambda exact: inputs.make_case(name="sc_fp8", seed=92, ctx_lens=PREFILL_LENS, n_q=PREFILL_NQ,
                                                     idx_dtype="fp8", n_heads_idx=19, head_dim_idx=64, topk=64,
                                                     sfa_dtype=None, exact=exact),
    "ragged_mxfp8": lambda exact: inputs.make_case(name="sc_mxfp8", seed=93, ctx_lens=PREFILL_LENS, n_q=PREFILL_NQ,
                                                   idx_dtype="mxfp8", n_heads_idx=37, head_dim_idx=128, topk=64,
                                                   sfa_dtype=None, exact=exact),
}


@pytest.mark.parametrize("name", sorted(SCORE_CASES))
@pytest.mark.parametrize("exact", [True, False], ids=["exact", "float"])
def test_indexer_scores(name, exact):
    case = parity.to_device(SCORE_CASES[name](exact))
    print(f"\n[case] scores {case.name} T={case.num_tokens}", flush=True)
    vis = oracle.visible(case.q_offsets.cpu().numpy(), case.ctx_lens.cpu().numpy())
    _, o_sc = parity.oracle_indexer(case)
    _, mag = parity.oracle_indexer(dataclasses.replace(case, weights=case.weights.abs()))
    first = None
    for route, flags in parity.indexer_routes(case).items():
        g = parity.gpu_indexer_scores(case, flags)
        print(route, parity.compare_scores(g, o_sc, vis, case.exact, mag, case.idx_dtype), flush=True)
        if first is None:
            first = g
        else:
            assert torch.equal(torch.nan_to_num(first, nan=7.0), torch.nan_to_num(g, nan=7.0)), route


# --- full-size workloads, checked on sampled rows -----------------------------
def _full(case, rows, routes=True):
    print(f"\n[case] {case.name} seed={case.seed} B={case.batch} T={case.num_tokens} "
          f"max_ctx={case.max_ctx} K={case.topk} rows={rows}", flush=True)
    idx = parity.gpu_indexer_topk(case)
    if routes:
        for name, flags in parity.indexer_routes(case).items():
            if flags:
                assert torch.equal(idx, parity.gpu_indexer_topk(case, flags=flags)), f"route {name} differs"
    out, _ = parity.gpu_sparse_attn(case, idx)
    stats = parity.check_rows(case, idx, out, rows)
    print(f"[ok] {case.name}: {stats}", flush=True)


def _seeded_rows(n_rows, count, seed, must=()):
    """`count` distinct seeded rows of n_rows, plus the `must` rows, sorted."""
    rng = np.random.default_rng(seed)
    rows = set(int(r) for r in must)
    rows |= set(int(r) for r in rng.choice(n_rows, size=min(count, n_rows), replace=False))
    return sorted(rows)


def _request_rows(case, requests):
    """Every query row of the given requests."""
    qo = case.q_offsets.cpu().tolist()
    return [i for b in requests for i in range(qo[b], qo[b + 1])]


def test_chunked_prefill_full():
    """4096 query rows appended to a 61440-token prefix (65536 positions):
    256 seeded rows, rows 0 and 4095 among them."""
    case = inputs.chunked_prefill(device="cuda")
    _full(case, _seeded_rows(4096, 254, 7, must=(0, 4095)))


def test_chunked_prefill_full_exact():
    """The chunked prefill in exact mode (integer inputs, every score an
    exact integer, many equal): index sets bit-exact on 64 seeded rows; each
    row's selection runs over 8 segments of 8192 positions with integer
    ties."""
    case = inputs.chunked_prefill(device="cuda", exact=True)
    _full(case, _seeded_rows(4096, 62, 8, must=(0, 4095)))


def test_scratch_prefill_full():
    """A prefill from scratch: 16384 causal query rows, row i sees i + 1 positions."""
    case = inputs.chunked_prefill(device="cuda", prefix=0, new=16384, name="prefill_0+16384_bf16")
    _full(case, [0, 1, 7, 8, 2046, 2047, 2048, 9001, 16383])


@pytest.mark.parametrize("batch", [1, 64])
def test_decode_32k_fp8_latent_full(batch):
    """The 32K decode with the fp8 latent cache, one and 64 requests."""
    case = inputs.decode_32k(batch=batch, device="cuda", sfa_dtype="fp8", name=f"decode_32k_kv8_b{batch}")
    _full(case, [0] if batch == 1 else [0, 31, 63], routes=False)


def test_spec_verify_full():
    """16 requests x 4 causal query rows at 262144 positions, fp8 indexer:
    every row of 4 requests and a seeded sample of the rest."""
    case = inputs.spec_verify(device="cuda")
    rows = sorted(set(_request_rows(case, [0, 5, 10, 15])) | set(_seeded_rows(64, 6, 9)))
    _full(case, rows, routes=False)


def test_spec_verify_full_exact():
    """The speculative-verify shape in exact mode: index sets bit-exact on
    every row of 4 requests and a seeded sample (32 segments of 8192
    positions per row, integer ties)."""
    case = inputs.spec_verify(device="cuda", exact=True)
    rows = sorted(set(_request_rows(case, [1, 6, 11, 14])) | set(_seeded_rows(64, 4, 10)))
    _full(case, rows, routes=False)


def test_spec_verify_mxfp8_full():
    """The speculative-verify shape with an MXFP8 indexer: 16 requests x 4
    causal rows at 262144 positions (two-pass route, four rows per key read)."""
    case = inputs.spec_verify(device="cuda", idx_dtype="mxfp8", name="spec_verify_mxfp8")
    _full(case, [0, 3, 17, 38, 60, 63], routes=False)


def test_prefill_mxfp8_full():
    """The chunked prefill (4096 rows over 65536 positions) with an MXFP8
    indexer: the row-tiled kernel at full size, every route."""
    case = inputs.chunked_prefill(device="cuda", idx_dtype="mxfp8", name="prefill_61440+4096_mxfp8")
    _full(case, [0, 1, 1000, 2047, 3333, 4095])


@pytest.mark.parametrize("wide", [False, True], ids=["narrow", "wide"])
def test_batched_fp8_full(wide):
    """64 single-row requests, lengths uniform in [4096, 131072], fp8 indexer:
    the longest and shortest requests, 4 fixed ones and a seeded sample."""
    case = inputs.batched_decode_fp8(wide=wide, device="cuda")
    lens = case.ctx_lens.cpu()
    rows = sorted({0, 63, int(lens.argmax()), int(lens.argmin()), 21, 42} | set(_seeded_rows(64, 6, 11)))
    _full(case, rows)


def test_batched_fp8_wide_full_exact():
    """The wide batched fp8 decode in exact mode: bit-exact index sets on a
    seeded sample of rows, the longest (two-pass selection) among them."""
    case = inputs.batched_decode_fp8(wide=True, device="cuda", exact=True)
    lens = case.ctx_lens.cpu()
    _full(case, sorted({int(lens.argmax()), int(lens.argmin())} | set(_seeded_rows(64, 6, 12))), routes=False)


def test_position_tiled_many_chunks_per_workgroup():
    """160 single-row requests at 262144 positions with a narrow fp8 indexer
    (4 x 64): 163840 chunks of 256 positions over 512 scoring workgroups,
    320 each, so every workgroup stages the block-table entries of its
    chunks in two windows (256, then 64) and restarts its tile ring between
    them; the rows at both ends of the batch against the oracle."""
    case = inputs.make_case(name="many_chunks_fp8_4x64", seed=97, ctx_lens=[262144] * 160, idx_dtype="fp8",
                            n_heads_idx=4, head_dim_idx=64, topk=2048, sfa_dtype=None, device="cuda")
    print(f"\n[case] {case.name} seed={case.seed} B={case.batch} T={case.num_tokens} "
          f"max_ctx={case.max_ctx} K={case.topk}", flush=True)
    idx = parity.gpu_indexer_topk(case)
    stats = parity.check_rows(case, idx, None, [0, 1, 63, 64, 158, 159])
    print(f"[ok] {case.name}: {stats}", flush=True)


# --- batched decode through the single-kernel indexer ---------------------------
# Many 256-position chunks per workgroup switch the fused kernel to its
# throughput modes (block-table entries in LDS, three key tiles in flight,
# keys staged in LDS when they fit); each case checks the indices against the
# two-pass route bit for bit and against the oracle on sampled rows.
def _fused_b24():
    rng = np.random.default_rng(91)
    lens = rng.integers(5000, 32769, size=24).tolist()
    n_q = [1 + (i % 3 == 0) for i in range(24)]
    return inputs.make_case(name="fused_b24_fp8_48h", seed=91, ctx_lens=lens, n_q=n_q, idx_dtype="fp8",
                            n_heads_idx=48, head_dim_idx=128, topk=2048, sfa_dtype=None, device="cuda")


FUSED_BATCHED = {
    # 64 one-row requests at 32768, 64 heads: the one-row 64-head mode, keys staged
    "b64_bf16": lambda: inputs.decode_32k(batch=64, device="cuda", sfa_dtype=None),
    # 24 requests of 1-2 rows, 48 fp8 heads, ragged lengths: the general batched mode
    "b24_fp8_48h": _fused_b24,
    # 300 requests: one workgroup each, more keys than LDS staging holds
    "b300_fp8_d64": lambda: inputs.make_case(name="fused_b300_fp8_d64", seed=92, ctx_lens=[20000] * 300, n_q=1,
                                             idx_dtype="fp8", n_heads_idx=64, head_dim_idx=64, topk=2048,
                                             sfa_dtype=None, device="cuda"),
    # MXFP8 keys: 64 one-row requests (one-row 64-head mode) and the general mode
    "b64_mxfp8": lambda: inputs.decode_32k(batch=64, device="cuda", sfa_dtype=None, idx_dtype="mxfp8",
                                           name="fused_b64_mxfp8"),
    # 4-row requests (speculative-verify shape) in the batched modes: the key
    # staging must fit the device's LDS beside 4 rows of staged queries
    "b32x4_bf16": lambda: inputs.decode_32k(batch=32, n_q=4, device="cuda", sfa_dtype=None,
                                            name="fused_b32x4_bf16"),
    "b64x4_bf16_16k": lambda: inputs.decode_32k(batch=64, n_q=4, ctx_lens=[16384] * 64, device="cuda",
                                                sfa_dtype=None, name="fused_b64x4_bf16_16k"),
    "b32x4_f32_64x64": lambda: inputs.make_case(name="fused_b32x4_f32_64x64", seed=98, ctx_lens=[32768] * 32,
                                                n_q=4, idx_dtype="f32", n_heads_idx=64, head_dim_idx=64,
                                                topk=2048, sfa_dtype=None, device="cuda"),
    "b24_mxfp8_48h": lambda: inputs.make_case(name="fused_b24_mxfp8_48h", seed=94,
                                              ctx_lens=[5000 + 1117 * i for i in range(24)],
                                              n_q=[1 + (i % 3 == 0) for i in range(24)], idx_dtype="mxfp8",
                                              n_heads_idx=48, head_dim_idx=128, topk=2048, sfa_dtype=None,
                                              device="cuda"),
}


@pytest.mark.parametrize("name", sorted(FUSED_BATCHED))
def test_fused_batched_modes(name):
    case = FUSED_BATCHED[name]()
    print(f"\n[case] {case.name} seed={case.seed} B={case.batch} T={case.num_tokens} "
          f"max_ctx={case.max_ctx} K={case.topk}", flush=True)
    idx = parity.gpu_indexer_topk(case)
    two = parity.gpu_indexer_topk(case, flags=parity.dsa.INDEXER_TWO_PASS)
    assert torch.equal(idx, two), "fused and two-pass indices differ"
    T = case.num_tokens
    rows = sorted({0, 1, T // 3, T // 2, T - 2, T - 1})
    stats = parity.check_rows(case, idx, None, rows)
    print(f"[ok] {case.name}: {stats}", flush=True)


def test_causal_planted_future_keys_never_selected():
    """Keys after a row's position made huge must never be selected."""
    case = inputs.spec_verify(batch=1, ctx=3000, exact=True)
    bt = case.block_table
    k = case.k_cache.clone()
    for t in range(2997, 3000):
        k[bt[0, t // 64], t % 64] = 0x70  # e4m3 code of 128
    q = case.q_idx.view(torch.float8_e4m3fn).float().abs().to(torch.float8_e4m3fn).view(torch.uint8)
    w = case.weights.abs() + 1
    import dataclasses
    case = dataclasses.replace(case, k_cache=k, q_idx=q.contiguous(), weights=w)
    _, _ = _run(case)
    idx = parity.gpu_indexer_topk(parity.to_device(case)).cpu()
    for j in range(4):
        pos = 2996 + j
        row = set(idx[j][idx[j] >= 0].tolist())
        assert max(row) <= pos
        assert {t for t in range(2997, 3000) if t <= pos} <= row


def test_all_ties_keep_the_lowest_positions():
    """Every key equal: each row's scores tie, its boundary bin holds all its
    positions (more than the segmented selection's candidate list, so the
    two-pass route selects those rows whole in one workgroup), and the tie
    rule keeps positions 0 .. K-1 on every route."""
    import dataclasses
    case = inputs.decode_32k(ctx_lens=[20000, 9000], n_q=[1, 3], topk=2048, exact=True)
    ones = torch.ones(case.k_cache.shape, dtype=torch.bfloat16)
    k = ones if case.k_cache.dtype == torch.bfloat16 else ones.view(case.k_cache.dtype)
    case = parity.to_device(dataclasses.replace(case, k_cache=k.contiguous()))
    qo, lens = case.q_offsets.cpu().numpy(), case.ctx_lens.cpu().numpy()
    K = case.topk
    for name, flags in {"default": 0, "two_pass": parity.dsa.INDEXER_TWO_PASS}.items():
        idx = parity.gpu_indexer_topk(case, flags=flags).cpu().numpy()
        for b in range(len(lens)):
            n = qo[b + 1] - qo[b]
            for j in range(n):
                vis = lens[b] - n + j + 1
                want = np.where(np.arange(K) < vis, np.arange(K), -1)
                assert np.array_equal(idx[qo[b] + j], want), f"{name}: request {b} row {j}"
        print(f"[ok] all ties, {name} route", flush=True)


@pytest.mark.parametrize("excess", [0, 100, -100], ids=["bin_taken_whole", "ties_past_k", "ties_below_k"])
def test_planted_ties_at_the_boundary(excess):
    """Two score values: every key is 1 except K + excess planted positions
    per request, whose keys are 2, with |q| and positive weights, so their
    scores are exactly twice the others and each group ties exactly.  With
    excess 0 the K-th key's bin holds exactly the keys needed (all of them
    tied), with 100 the tie rule drops the last 100 planted positions, and
    with -100 it keeps the lowest 100 unplanted positions."""
    case = inputs.decode_32k(ctx_lens=[20000, 9000], n_q=[1, 3], topk=2048, exact=True)
    K = case.topk
    bt = case.block_table
    kf = torch.ones(case.k_cache.shape, dtype=torch.float32)
    g = torch.Generator().manual_seed(4242)
    planted = []
    for b, span in enumerate([20000, 8998]):  # (request 1's earliest row sees 8998 positions)
        pos = torch.randperm(span, generator=g)[:K + excess].tolist()
        for t in pos:
            kf[bt[b, t // 64], t % 64] = 2.0
        planted.append(set(pos))
    kb = kf.to(torch.bfloat16)
    k = kb if case.k_cache.dtype == torch.bfloat16 else kb.view(case.k_cache.dtype)
    qv = case.q_idx if case.q_idx.dtype == torch.bfloat16 else case.q_idx.view(torch.bfloat16)
    qa = qv.float().abs().to(torch.bfloat16)
    q = qa if case.q_idx.dtype == torch.bfloat16 else qa.view(case.q_idx.dtype)
    case = parity.to_device(dataclasses.replace(case, k_cache=k.contiguous(), q_idx=q.contiguous(),
                                                weights=case.weights.abs() + 1))
    qo, lens = case.q_offsets.cpu().numpy(), case.ctx_lens.cpu().numpy()
    for name, flags in {"default": 0, "two_pass": parity.dsa.INDEXER_TWO_PASS}.items():
        idx = parity.gpu_indexer_topk(case, flags=flags).cpu().numpy()
        for b in range(len(lens)):
            n = qo[b + 1] - qo[b]
            for j in range(n):
                vis = int(lens[b] - n + j + 1)
                val = np.ones(vis, dtype=np.int64)
                val[[t for t in planted[b] if t < vis]] = 2
                order = np.lexsort((np.arange(vis), -val))  # higher value first, then lower position
                want = np.sort(order[:K])
                assert np.array_equal(idx[qo[b] + j], want), f"{name}: request {b} row {j}"
        print(f"[ok] planted ties excess={excess}, {name} route", flush=True)


# --- sparse attention alone, on the oracle's indices ---------------------------
def test_sfa_on_oracle_indices_with_padding():
    case = parity.to_device(inputs.decode_32k(ctx_lens=[9000, 1500, 200], n_q=[1, 2, 1], topk=1024))
    o_idx, _ = parity.oracle_indexer(case)
    o_idx[1, 700:] = -1     # a short list
    o_idx[2, :] = -1        # nothing selected
    g_out, g_lse = parity.gpu_sparse_attn(case, torch.from_numpy(o_idx).cuda())
    r_out, r_lse = parity.oracle_sfa(case, o_idx)
    print(parity.compare_out(g_out, r_out, "bf16", gpu_lse=g_lse, ora_lse=r_lse))
    assert np.all(parity.out_to_f64(g_out, "bf16")[2] == 0.0)


@pytest.mark.parametrize("heads", [16, 32, 48, 64, 80, 128])
def test_sfa_head_counts(heads):
    case = parity.to_device(inputs.make_case(name=f"sfa{heads}", seed=81, ctx_lens=[3000, 2500], n_q=[1, 3],
                                             idx_dtype="bf16", n_heads_idx=16, head_dim_idx=64, topk=512,
                                             sfa_dtype="bf16", n_heads_sfa=heads))
    idx = parity.gpu_indexer_topk(case)
    g_out, g_lse = parity.gpu_sparse_attn(case, idx)
    r_out, r_lse = parity.oracle_sfa(case, idx)
    print(parity.compare_out(g_out, r_out, "bf16", gpu_lse=g_lse, ora_lse=r_lse))


@pytest.mark.parametrize("name", ["tiny", "decode_32k", "spec_verify"])
def test_workspace_reuse_across_calls(name):
    """Many calls on one workspace: the fused indexer's arrival counters and
    the two-pass histograms must return to zero after every call."""
    from lightning_indexer_top_02_amd import dsa
    case = {"tiny": lambda: inputs.tiny_decode(),
            "decode_32k": lambda: inputs.decode_32k(ctx_lens=[32768, 5000], n_q=[1, 1]),
            "spec_verify": lambda: inputs.spec_verify(batch=3, ctx=9000)}[name]()
    case = parity.to_device(case)
    paged, idx = parity.paged_of(case), parity.indexer_of(case)
    ws = dsa.new_workspace(dsa.indexer_topk_workspace_size(paged, idx), "cuda")
    first = None
    for it in range(50):
        out = torch.empty((case.num_tokens, case.topk), dtype=torch.int32, device="cuda")
        dsa.indexer_topk(paged, idx, out, workspace=ws)
        if first is None:
            first = out.clone()
        else:
            assert torch.equal(out, first), f"call {it} differs"
    ctrl = ws[: 4 * case.batch].view(torch.int32)
    assert int(ctrl.abs().sum()) == 0, "arrival counters not back to zero"
    for flags in parity.indexer_routes(case).values():
        assert torch.equal(first, parity.gpu_indexer_topk(case, flags=flags))


# --- HIP graph capture: replays equal the eager result ------------------------
@pytest.mark.parametrize("flags", [0, 1], ids=["default_route", "two_pass"])
def test_graph_replays_match_eager(flags):
    """The step captured into a HIP graph and replayed several times, with
    eager calls on the same workspace and synchronisations between replays,
    gives the eager result every time (the workspace counters, histograms and
    candidate lists must be back to zero after each call)."""
    from lightning_indexer_top_02_amd import dsa
    case = parity.to_device(inputs.make_case(name="graph", seed=95, ctx_lens=[32768, 9000, 20000], n_q=[1, 1, 4],
                                             idx_dtype="bf16", n_heads_idx=64, head_dim_idx=128, topk=2048,
                                             sfa_dtype="bf16", n_heads_sfa=64))
    paged, idx = parity.paged_of(case), parity.indexer_of(case, flags=flags)
    out, lse = parity.sfa_tensors(case)
    sfa = dsa.make_sfa(case.q_sfa, case.kv_cache, out, case.scale, case.sfa_dtype, lse=lse)
    ws = dsa.new_workspace(dsa.fused_decode_workspace_size(paged, idx, sfa), "cuda")
    ii = torch.empty((case.num_tokens, case.topk), dtype=torch.int32, device="cuda")
    dsa.fused_decode(paged, idx, sfa, topk_idx=ii, workspace=ws)
    torch.cuda.synchronize()
    ref = (ii.clone(), out.clone(), lse.clone())
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        dsa.fused_decode(paged, idx, sfa, topk_idx=ii, workspace=ws, stream=cs)
    torch.cuda.synchronize()
    for rep in range(4):
        ii.fill_(-7)
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ii, ref[0]), f"replay {rep}: indices differ"
        assert torch.equal(out, ref[1]) and torch.equal(lse, ref[2]), f"replay {rep}: outputs differ"
        dsa.fused_decode(paged, idx, sfa, topk_idx=ii, workspace=ws)  # eager call between replays
        torch.cuda.synchronize()
        assert torch.equal(ii, ref[0]), f"eager call after replay {rep} differs"
    ctrl = ws[: 4 * case.batch].view(torch.int32)
    assert int(ctrl.abs().sum()) == 0, "arrival counters not back to zero"@pytest.mark.gpu
def test_decode_32k_batch8_full():
    """The 32K decode at batch 8: 16 attention splits per row, merged by two
    lanes per (row, head, 4 dims); three rows against the oracle."""
    case = inputs.decode_32k(batch=8, device="cuda", name="decode_32k_b8")
    _full(case, [0, 3, 7], routes=False)




"""GPU parity of the indexer cache append (dsa_indexer_cache_append) with the
CPU oracle: the whole pools after the append (new slots and untouched ones)
must be bit-identical, since every stored value is an integer decision (a
code, a scale, a rounded bf16) taken from the same fp32 values."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import parity
from lightning_indexer_top_02_amd import dsa, inputs

pytestmark = pytest.mark.gpu

SENTINEL = {"f32": (-7.0, None), "bf16": (0x1234, None), "fp8": (0x55, -1.0), "mxfp8": (0x55, 3)}
STORE = {"f32": torch.float32, "bf16": torch.int16, "fp8": torch.uint8, "mxfp8": torch.uint8}


def _pools(case, D, dst):
    fill, sfill = SENTINEL[dst]
    kc = torch.full((case.num_pages, 64, D), fill, dtype=STORE[dst])
    ks = None
    if dst == "fp8":
        ks = torch.full((case.num_pages, 64), sfill, dtype=torch.float32)
    elif dst == "mxfp8":
        ks = torch.full((case.num_pages, 64, D // 32), sfill, dtype=torch.uint8)
    return kc, ks


def _src(case, src):
    x = case.k_new.cpu()
    return x.contiguous() if src == "f32" else x.to(torch.bfloat16).view(torch.int16).contiguous()


def _gpu_append(case, src, dst, D):
    kc, ks = _pools(case, D, dst)
    kc, ks = kc.cuda(), None if ks is None else ks.cuda()
    k_new = _src(case, src).cuda()
    # the paging tensors stay referenced until the kernel has finished
    qo, lens, bt = case.q_offsets.cuda(), case.ctx_lens.cuda(), case.block_table.cuda()
    paged = dsa.make_paged(qo, lens, bt, case.num_pages, max_q_per_req=case.max_q_per_req, max_ctx_len=case.max_ctx)
    dsa.cache_append(paged, dsa.make_cache_append(k_new, src, kc, dst, k_scale=ks))
    torch.cuda.synchronize()
    del qo, lens, bt
    return kc.cpu(), None if ks is None else ks.cpu()


def _oracle_append(case, src, dst, D):
    kc, ks = _pools(case, D, dst)
    raw = inputs.to_numpy_raw(_src(case, src))
    return oracle.cache_append(case.q_offsets.numpy(), case.ctx_lens.numpy(), case.block_table.numpy(), 64,
                               src, raw, dst, inputs.to_numpy_raw(kc), inputs.to_numpy_raw(ks))


def _check(case, src, dst, D):
    print(f"\n[case] append {case.name} src={src} dst={dst} D={D} T={case.k_new.shape[0]}", flush=True)
    g_kc, g_ks = _gpu_append(case, src, dst, D)
    o_kc, o_ks = _oracle_append(case, src, dst, D)
    g = inputs.to_numpy_raw(g_kc)
    bad = np.argwhere(g.view(np.uint8) != np.ascontiguousarray(o_kc).view(np.uint8))
    assert bad.size == 0, f"cache differs from the oracle at {bad[:4].tolist()}"
    if o_ks is not None:
        gs = inputs.to_numpy_raw(g_ks)
        assert np.array_equal(gs.view(np.uint8), np.ascontiguousarray(o_ks).view(np.uint8)), "scales differ"
    print(f"[ok] append {case.name} {src}->{dst}", flush=True)


# Ragged requests: a 1-token request, keys crossing page boundaries, a whole
# page, 200 keys at the end of a 1000-token request, directed rows (zeros,
# e4m3 midpoints, fp32-quotient midpoints).
LENS, NQ = [1, 70, 64, 1000, 300], [1, 3, 64, 200, 17]
COMBOS = [(s, d, D) for s in ("f32", "bf16") for d in ("f32", "bf16", "fp8", "mxfp8") for D in (64, 128)
          if not (d == "mxfp8" and D == 64)]


@pytest.mark.parametrize("src,dst,D", COMBOS, ids=[f"{s}-{d}-{D}" for s, d, D in COMBOS])
def test_cache_append_matches_oracle(src, dst, D):
    _check(inputs.append_case(31, LENS, NQ, D, name="ragged"), src, dst, D)


@pytest.mark.parametrize("dst", ["fp8", "mxfp8"])
def test_cache_append_full_prefill_and_decode(dst):
    """The chunked-prefill append (4096 keys at 61440..65535) and a 64-request
    decode append (one key each at lengths up to 131072), as the step appends
    them, checked whole."""
    _check(inputs.append_case(32, [65536], [4096], 128, name="prefill_61440+4096"), "f32", dst, 128)
    lens = inputs.batched_fp8_lengths(seed=33)
    _check(inputs.append_case(33, lens, 1, 128, name="decode_b64"), "bf16", dst, 128)


@pytest.mark.parametrize("dst", ["fp8", "mxfp8"])
def test_appended_cache_feeds_the_indexer(dst):
    """The indexer reading a cache the GPU appended gives the same indices as
    on the oracle-appended cache, and those match the oracle's indexer."""
    base = inputs.make_case(name=f"append_then_score_{dst}", seed=34, ctx_lens=[3000, 700], n_q=[4, 64],
                            idx_dtype=dst, n_heads_idx=64, head_dim_idx=128, topk=256, sfa_dtype=None)
    ap = inputs.append_case(35, [3000, 700], [4, 64], 128, name="append_then_score")
    # the new keys go into the case's own pages (its block table), over its data
    kc = base.k_cache.clone().cuda()
    ks = base.k_scale.clone().cuda()
    dev = parity.to_device(base)  # referenced until the end: the paging pointers live in it
    k_new = ap.k_new.cuda()
    paged = parity.paged_of(dev)
    dsa.cache_append(paged, dsa.make_cache_append(k_new, "f32", kc, dst, k_scale=ks))
    o_kc, o_ks = oracle.cache_append(base.q_offsets.numpy(), base.ctx_lens.numpy(), base.block_table.numpy(), 64,
                                     "f32", ap.k_new.numpy(), dst, base.k_cache.numpy(), base.k_scale.numpy())
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), o_kc) and np.array_equal(ks.cpu().numpy().view(np.uint8),
                                                                     np.ascontiguousarray(o_ks).view(np.uint8))
    case = dataclasses.replace(dev, k_cache=kc, k_scale=ks)
    idx = parity.gpu_indexer_topk(case)
    stats = parity.check_rows(case, idx, None, list(range(case.num_tokens)))
    print(f"[ok] {base.name}: {stats}", flush=True)


def test_cache_append_graph_replays_match_eager():
    """The append captured in a HIP graph: three replays, each after the pools
    are reset eagerly, every one equal to the eager append."""
    case = inputs.append_case(36, LENS, NQ, 128, name="graph")
    qo, lens, bt = case.q_offsets.cuda(), case.ctx_lens.cuda(), case.block_table.cuda()
    paged = dsa.make_paged(qo, lens, bt, case.num_pages, max_q_per_req=case.max_q_per_req, max_ctx_len=case.max_ctx)
    k_new = case.k_new.cuda()
    kc0, ks0 = (t.cuda() for t in _pools(case, 128, "mxfp8"))
    kc, ks = kc0.clone(), ks0.clone()
    ap = dsa.make_cache_append(k_new, "f32", kc, "mxfp8", k_scale=ks)
    dsa.cache_append(paged, ap)
    torch.cuda.synchronize()
    ref_c, ref_s = kc.clone(), ks.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dsa.cache_append(paged, ap, stream=side)
    torch.cuda.synchronize()
    for rep in range(3):
        kc.copy_(kc0)
        ks.copy_(ks0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(kc, ref_c) and torch.equal(ks, ref_s), f"replay {rep} differs from the eager append"
    del g
    print("[ok] append graph replays", flush=True)


# --- latent rows (dsa_latent_cache_append) --------------------------------------
LATENT_SENTINEL = {"f32": -7.0, "bf16": 0x1234, "fp8": 0x55}
LATENT_ROW = {"f32": 576, "bf16": 576, "fp8": 656}


def _latent_case(seed=37, lens=LENS, nq=NQ, name="latent_ragged"):
    """Ragged new latent rows, with directed rows at the fp8 tile-exponent
    boundaries: a tile whose amax is exactly 448 * 2^3 (exponent 3) and one
    just above it (exponent 4), a tile of 1e-38 (exponent clamped to -126),
    a zero row, e4m3 midpoints with 448 in every 32-block (exponent 0)."""
    c = inputs.append_case(seed, lens, nq, 576, name=name)
    x = c.k_new.clone()
    if x.shape[0] >= 12:
        x[6:10] = x[6:10].clamp(-3, 3)
        x[6, 5] = 448.0 * 8
        x[7, 130] = float(np.nextafter(np.float32(448.0 * 8), np.float32(1e9)))
        x[8, 256:384] = 1e-38
        x[9] = 0.0
    return dataclasses.replace(c, k_new=x.contiguous())


def _latent_pool(case, dst):
    dt = torch.float32 if dst == "f32" else (torch.int16 if dst == "bf16" else torch.uint8)
    return torch.full((case.num_pages, 64, LATENT_ROW[dst]), LATENT_SENTINEL[dst], dtype=dt)


def _check_latent(case, src, dst):
    print(f"\n[case] latent append {case.name} src={src} dst={dst} T={case.k_new.shape[0]}", flush=True)
    kv = _latent_pool(case, dst).cuda()
    x_new = _src(case, src).cuda()
    qo, lens, bt = case.q_offsets.cuda(), case.ctx_lens.cuda(), case.block_table.cuda()
    paged = dsa.make_paged(qo, lens, bt, case.num_pages, max_q_per_req=case.max_q_per_req, max_ctx_len=case.max_ctx)
    dsa.latent_append(paged, dsa.make_latent_append(x_new, src, kv, dst))
    torch.cuda.synchronize()
    del qo, lens, bt
    o = oracle.latent_append(case.q_offsets.numpy(), case.ctx_lens.numpy(), case.block_table.numpy(), 64, src,
                             inputs.to_numpy_raw(_src(case, src)), dst, inputs.to_numpy_raw(_latent_pool(case, dst)))
    g = inputs.to_numpy_raw(kv.cpu())
    bad = np.argwhere(g.view(np.uint8) != np.ascontiguousarray(o).view(np.uint8))
    assert bad.size == 0, f"latent pool differs from the oracle at {bad[:4].tolist()}"
    print(f"[ok] latent append {case.name} {src}->{dst}", flush=True)


LATENT_COMBOS = [(s, d) for s in ("f32", "bf16") for d in ("f32", "bf16", "fp8")]


@pytest.mark.parametrize("src,dst", LATENT_COMBOS, ids=[f"{s}-{d}" for s, d in LATENT_COMBOS])
def test_latent_append_matches_oracle(src, dst):
    _check_latent(_latent_case(), src, dst)


def test_latent_append_decode_batch_fp8():
    """A 64-request decode append (one row each, lengths up to 131072) into
    fp8 latent rows, checked whole."""
    lens = inputs.batched_fp8_lengths(seed=38)
    _check_latent(_latent_case(38, lens, 1, name="latent_decode_b64"), "bf16", "fp8")


@pytest.mark.parametrize("sfa_dtype", ["bf16", "fp8"])
def test_two_stream_appends_then_decode(sfa_dtype):
    """The step's producers on two streams at once: the indexer-key append on
    one, the latent-row append on the other, joined by events before the
    fused decode on the caller's stream.  The pools equal the oracle's
    appends bit for bit, and the decode over them matches the oracle."""
    base = inputs.make_case(name=f"two_stream_{sfa_dtype}", seed=39, ctx_lens=[3000, 700, 4500], n_q=[1, 4, 2],
                            idx_dtype="bf16", n_heads_idx=64, head_dim_idx=128, topk=512, sfa_dtype=sfa_dtype,
                            n_heads_sfa=128)
    g = torch.Generator()
    g.manual_seed(40)
    T = base.num_tokens
    k_new = torch.randn((T, 128), generator=g)
    x_new = torch.randn((T, 576), generator=g) * 0.5
    dev = parity.to_device(base)  # referenced until the end: the paging pointers live in it
    kc, kv = dev.k_cache.clone(), dev.kv_cache.clone()
    paged = parity.paged_of(dev)
    kn, xn = k_new.cuda(), x_new.cuda()
    ak = dsa.make_cache_append(kn, "f32", kc, "bf16")
    al = dsa.make_latent_append(xn, "f32", kv, sfa_dtype)
    cur = torch.cuda.current_stream()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(cur)
    s2.wait_stream(cur)
    dsa.cache_append(paged, ak, stream=s1)
    dsa.latent_append(paged, al, stream=s2)
    cur.wait_stream(s1)
    cur.wait_stream(s2)
    case = dataclasses.replace(dev, k_cache=kc, kv_cache=kv)
    f_idx, f_out, f_lse = parity.gpu_fused_decode(case)
    torch.cuda.synchronize()
    args = (base.q_offsets.numpy(), base.ctx_lens.numpy(), base.block_table.numpy(), 64, "f32")
    o_kc, _ = oracle.cache_append(*args, k_new.numpy(), "bf16", inputs.to_numpy_raw(base.k_cache))
    o_kv = oracle.latent_append(*args, x_new.numpy(), sfa_dtype, inputs.to_numpy_raw(base.kv_cache))
    assert np.array_equal(inputs.to_numpy_raw(kc.cpu()), o_kc), "indexer pool differs from the oracle's append"
    assert np.array_equal(inputs.to_numpy_raw(kv.cpu()), o_kv), "latent pool differs from the oracle's append"
    stats = parity.check_case(case)
    print(f"[ok] {base.name}: {stats}", flush=True)
    s_idx, s_out, _ = parity.gpu_fused_decode(case)
    assert torch.equal(f_idx, s_idx) and torch.equal(f_out, s_out)

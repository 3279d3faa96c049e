"""Seeded synthetic inputs for the DSA sparse-attention step.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests.  It holds no arithmetic of the method itself (no scoring, no
selection, no attention): it draws random tensors, casts them to their storage
types, quantizes the fp8 route's inputs the way the step's producer would, and
lays them out in a paged pool behind a shuffled block table.

Workload shapes follow the paged-cache problem statement the pages give for the
indexer and the sparse attention kernel ("Day0 Inference Support and
Performance Optimization for New LLM Architectures", section III, 3.1 and 3.2):
a paged K cache and block table, query and per-head weights, and the MLA
latent cache.  Pages hold 64 tokens.  Pool pages that no request maps
("decoys"), slots past a request's length in its last page, and block-table
entries past a request's last page point at NaN data, so any stray read poisons
the result instead of passing silently.

Storage conventions: fp32 values as float32, bf16 as its 16-bit pattern,
fp8 e4m3 (OCP, no infinities) as its 8-bit code with an fp32 scale (one per
(query row, head) for q, one per cached token for k).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

PAGE_SIZE = 64
QK_DIM = 576  # 512 latent + 64 rope
V_DIM = 512
FP8_MAX = 448.0

DTYPE_CODE = {"f32": 0, "bf16": 1, "fp8": 2, "mxfp8": 3}


@dataclasses.dataclass
class Case:
    """One batch of DSA-step inputs.  Tensors live on ``device``."""

    name: str
    seed: int
    exact: bool
    page_size: int
    # paging
    q_offsets: torch.Tensor  # int32 [B+1]
    ctx_lens: torch.Tensor  # int32 [B]
    block_table: torch.Tensor  # int32 [B][max_pages]
    num_pages: int
    decoy_pages: torch.Tensor  # int64 [n_decoy]
    # indexer
    idx_dtype: str
    n_heads_idx: int
    head_dim_idx: int
    topk: int
    q_idx: torch.Tensor  # [T][H_I][D_I] float32 | int16 (bf16 bits) | uint8 (e4m3 codes)
    q_scale: Optional[torch.Tensor]  # float32 [T][H_I] (fp8 only)
    weights: torch.Tensor  # float32 [T][H_I]
    k_cache: torch.Tensor  # [num_pages][64][D_I] raw storage
    k_scale: Optional[torch.Tensor]  # fp8: float32 [num_pages][64]; mxfp8: uint8 E8M0 [num_pages][64][D_I/32]
    # sparse attention
    sfa_dtype: str
    n_heads_sfa: int
    qk_dim: int
    v_dim: int
    scale: float
    q_sfa: Optional[torch.Tensor]  # [T][H_q][576] raw storage
    kv_cache: Optional[torch.Tensor]  # [num_pages][64][576] raw storage

    @property
    def batch(self) -> int:
        return int(self.ctx_lens.numel())

    @property
    def num_tokens(self) -> int:
        return int(self.q_offsets[-1].item())

    @property
    def max_ctx(self) -> int:
        return int(self.ctx_lens.max().item())

    @property
    def max_q_per_req(self) -> int:
        return int((self.q_offsets[1:] - self.q_offsets[:-1]).max().item())


def _bf16_bits(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16).view(torch.int16)


def _nan_like_storage(dtype: str, shape, device) -> torch.Tensor:
    if dtype == "f32":
        return torch.full(shape, float("nan"), dtype=torch.float32, device=device)
    if dtype == "bf16":
        return torch.full(shape, 0x7FC0, dtype=torch.int16, device=device)
    return torch.full(shape, 0x7F, dtype=torch.uint8, device=device)


def quantize_e4m3_rows(x: torch.Tensor):
    """Producer-side fp8 quantization of an input tensor along its last dim:
    scale = amax / 448 per row, codes = saturating round-to-nearest-even cast.
    Returns (uint8 codes, float32 scales).  Rows of zeros get scale 1."""
    amax = x.abs().amax(dim=-1, keepdim=True).float()
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    codes = (x.float() / scale).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8), scale.squeeze(-1).contiguous()


def quantize_mxfp8(x: torch.Tensor):
    """Producer-side MXFP8 quantization along the last dim (OCP microscaling,
    blocks of 32 elements): the block's shared exponent is
    floor(log2(amax)) - 8 (8 = the largest e4m3 exponent), stored biased by
    127 as an E8M0 byte; codes = saturating round-to-nearest-even e4m3 casts
    of x / 2^exponent.  Blocks of zeros get exponent 0 (byte 127).  Returns
    (uint8 codes [..., D], uint8 E8M0 bytes [..., D/32])."""
    shp = x.shape
    xb = x.float().reshape(*shp[:-1], shp[-1] // 32, 32)
    amax = xb.abs().amax(dim=-1, keepdim=True)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax.clamp_min(1e-38))) - 8, torch.zeros_like(amax))
    e = e.clamp(-127, 127)
    codes = (xb / torch.exp2(e)).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8).reshape(shp), (e.squeeze(-1) + 127).to(torch.uint8).contiguous()


def pack_latent_fp8(x: torch.Tensor, v_dim: int = V_DIM, unit_scales: bool = False) -> torch.Tensor:
    """Producer-side fp8 latent rows: the first v_dim elements as e4m3 codes
    with one power-of-two scale per 128-element tile, 2^e with e the smallest
    integer such that amax / 2^e <= 448 (e = 0 for a zero tile, or throughout
    with ``unit_scales``; clamped to [-126, 127]), codes = nearest-even casts
    of x / 2^e (saturating); then a 16-byte block holding the tiles' E8M0
    bytes e + 127; then the remaining (rope) elements as bf16.  Returns uint8
    rows of v_dim + 16 + 2 (dim - v_dim) bytes."""
    lead, dim = x.shape[:-1], x.shape[-1]
    tiles = x[..., :v_dim].float().reshape(*lead, v_dim // 128, 128)
    amax = tiles.abs().amax(dim=-1, keepdim=True)
    e = torch.where(amax > 0, torch.ceil(torch.log2(amax.clamp_min(1e-38) / FP8_MAX)), torch.zeros_like(amax))
    if unit_scales:
        e = torch.zeros_like(e)
    e = e.clamp(-126, 127)
    codes = (tiles / torch.exp2(e)).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    codes = codes.reshape(*lead, v_dim)
    eblock = torch.zeros((*lead, 16), dtype=torch.uint8, device=x.device)
    eblock[..., : v_dim // 128] = (e.squeeze(-1) + 127).to(torch.uint8)
    rope = _bf16_bits(x[..., v_dim:].float()).contiguous().view(torch.uint8)
    return torch.cat([codes, eblock, rope], dim=-1).contiguous()


def _draw(gen, shape, device, dist: str, std: float = 1.0, exact: bool = False):
    if exact:
        return torch.randint(-3, 4, shape, generator=gen, device=device).float()
    if dist == "normal":
        return torch.randn(shape, generator=gen, device=device) * std
    if dist == "uniform":
        return torch.rand(shape, generator=gen, device=device)
    raise ValueError(dist)


def _storage(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x.float().contiguous()
    if dtype == "bf16":
        return _bf16_bits(x).contiguous()
    raise ValueError(dtype)


def make_case(
    *,
    name: str = "custom",
    seed: int,
    ctx_lens,
    n_q=1,
    idx_dtype: str = "bf16",
    n_heads_idx: int = 64,
    head_dim_idx: int = 128,
    topk: int = 2048,
    w_dist: str = "normal8",
    idx_std: float = 1.0,
    sfa_dtype: Optional[str] = "bf16",
    n_heads_sfa: int = 128,
    sfa_std: float = 0.5,
    qk_dim: int = QK_DIM,
    v_dim: int = V_DIM,
    scale: Optional[float] = None,
    exact: bool = False,
    n_decoy: int = 8,
    shuffle: bool = True,
    page_size: int = PAGE_SIZE,
    device="cpu",
) -> Case:
    """Draw one seeded case.

    ctx_lens: per-request cached lengths L_b (each includes its n_q query tokens).
    n_q: query tokens per request (int, or one per request).
    w_dist: "uniform" (U(0,1)) or "normal8" (N(0,1)/8) for the head weights.
    exact: every input is an integer in [-3, 3] (fp8 scales are 1), so every
           score is an exact small integer in fp32 and fp64 alike.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    ctx = [int(x) for x in ctx_lens]
    B = len(ctx)
    nq = [int(n_q)] * B if np.isscalar(n_q) else [int(x) for x in n_q]
    assert len(nq) == B and all(1 <= nq[b] <= ctx[b] for b in range(B))
    q_offsets = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    T = int(q_offsets[-1])

    # ---- paging: pages for every request + decoys, globally shuffled -------
    pages_per_req = [(L + page_size - 1) // page_size for L in ctx]
    n_mapped = sum(pages_per_req)
    num_pages = n_mapped + n_decoy
    cpu_gen = torch.Generator()
    cpu_gen.manual_seed(int(seed) + 7919)
    perm = torch.randperm(num_pages, generator=cpu_gen) if shuffle else torch.arange(num_pages)
    max_pages = max(pages_per_req)
    decoys = perm[n_mapped:].clone()
    bt = torch.empty((B, max_pages), dtype=torch.int32)
    # unused block-table entries point at a decoy page (NaN data) when one exists
    bt.fill_(int(decoys[0]) if n_decoy > 0 else 0)
    cur = 0
    for b in range(B):
        bt[b, : pages_per_req[b]] = perm[cur : cur + pages_per_req[b]].to(torch.int32)
        cur += pages_per_req[b]

    # ---- indexer inputs -----------------------------------------------------
    H, D = n_heads_idx, head_dim_idx
    w_kind = "uniform" if w_dist == "uniform" else "normal"
    w = _draw(gen, (T, H), device, w_kind, 1.0, exact)
    if not exact and w_dist == "normal8":
        w = w / 8.0
    w = w.float().contiguous()

    q_val = _draw(gen, (T, H, D), device, "normal", idx_std, exact)
    k_val = _draw(gen, (num_pages, page_size, D), device, "normal", idx_std, exact)
    if idx_dtype == "fp8":
        if exact:
            q_idx = q_val.to(torch.float8_e4m3fn).view(torch.uint8)
            k_cache = k_val.to(torch.float8_e4m3fn).view(torch.uint8)
            q_scale = torch.ones((T, H), dtype=torch.float32, device=device)
            k_scale = torch.ones((num_pages, page_size), dtype=torch.float32, device=device)
        else:
            q_idx, q_scale = quantize_e4m3_rows(q_val)
            k_cache, k_scale = quantize_e4m3_rows(k_val)
        k_scale = k_scale.clone()
    elif idx_dtype == "mxfp8":
        if exact:  # integer codes, unit block scales (E8M0 byte 127)
            q_idx = q_val.to(torch.float8_e4m3fn).view(torch.uint8)
            k_cache = k_val.to(torch.float8_e4m3fn).view(torch.uint8)
            q_scale = torch.full((T, H, D // 32), 127, dtype=torch.uint8, device=device)
            k_scale = torch.full((num_pages, page_size, D // 32), 127, dtype=torch.uint8, device=device)
        else:
            q_idx, q_scale = quantize_mxfp8(q_val)
            k_cache, k_scale = quantize_mxfp8(k_val)
        k_scale = k_scale.clone()
    else:
        q_idx, k_cache = _storage(q_val, idx_dtype), _storage(k_val, idx_dtype)
        q_scale = k_scale = None
    del q_val, k_val

    # ---- sparse-attention inputs -------------------------------------------
    q_sfa = kv_cache = None
    if sfa_dtype is not None:
        q_store = "bf16" if sfa_dtype == "fp8" else sfa_dtype  # the fp8 latent route takes bf16 queries
        q_sfa = _storage(_draw(gen, (T, n_heads_sfa, qk_dim), device, "normal", sfa_std, exact), q_store)
        lat = _draw(gen, (num_pages, page_size, qk_dim), device, "normal", sfa_std, exact)
        kv_cache = pack_latent_fp8(lat, v_dim, unit_scales=exact) if sfa_dtype == "fp8" else _storage(lat, sfa_dtype)

    # ---- poison everything no correct read touches -------------------------
    poison_pages = decoys.to(device)
    if n_decoy > 0:
        k_cache[poison_pages] = _nan_like_storage(idx_dtype, k_cache[poison_pages].shape, device)
        if k_scale is not None:
            k_scale[poison_pages] = float("nan") if k_scale.dtype == torch.float32 else 255
        if kv_cache is not None:
            kv_cache[poison_pages] = _nan_like_storage(sfa_dtype, kv_cache[poison_pages].shape, device)
    for b in range(B):
        tail = ctx[b] % page_size
        if tail:
            last = int(bt[b, pages_per_req[b] - 1])
            k_cache[last, tail:] = _nan_like_storage(idx_dtype, k_cache[last, tail:].shape, device)
            if k_scale is not None:
                k_scale[last, tail:] = float("nan") if k_scale.dtype == torch.float32 else 255
            if kv_cache is not None:
                kv_cache[last, tail:] = _nan_like_storage(sfa_dtype, kv_cache[last, tail:].shape, device)

    return Case(
        name=name, seed=int(seed), exact=bool(exact), page_size=page_size,
        q_offsets=torch.from_numpy(q_offsets).to(device),
        ctx_lens=torch.tensor(ctx, dtype=torch.int32, device=device),
        block_table=bt.to(device), num_pages=num_pages, decoy_pages=decoys,
        idx_dtype=idx_dtype, n_heads_idx=H, head_dim_idx=D, topk=int(topk),
        q_idx=q_idx.contiguous(), q_scale=q_scale, weights=w, k_cache=k_cache.contiguous(),
        k_scale=k_scale,
        sfa_dtype=sfa_dtype or "none", n_heads_sfa=n_heads_sfa, qk_dim=qk_dim, v_dim=v_dim,
        scale=float(scale if scale is not None else 1.0 / math.sqrt(qk_dim)),
        q_sfa=q_sfa, kv_cache=kv_cache,
    )


# ---------------------------------------------------------------------------
# The five workloads.  Lengths for the batched route are integer-uniform and
# inclusive, drawn from the seed.
# ---------------------------------------------------------------------------
def tiny_decode(seed=1001, exact=False, device="cpu", **kw):
    """Batch 1, context 4096, fp32 indexer 4 heads x 64, Top-K 256, fp32 sparse
    attention with 16 heads over the 512+64 latent cache, w ~ U(0,1)."""
    args = dict(name="tiny_decode_4k_f32" + ("_exact" if exact else ""), seed=seed,
                ctx_lens=[4096], n_q=1, idx_dtype="f32", n_heads_idx=4, head_dim_idx=64,
                topk=256, w_dist="uniform", sfa_dtype="f32", n_heads_sfa=16, sfa_std=1.0,
                exact=exact, device=device)
    args.update(kw)
    return make_case(**args)


def decode_32k(seed=1002, exact=False, batch=1, device="cpu", **kw):
    """Single-request decode at 32768 context: bf16 indexer 64 heads x 128,
    Top-K 2048, bf16 sparse attention with 128 heads, w ~ N(0,1)/8, latent
    cache ~ N(0, 0.5^2).  ``batch`` > 1 repeats the shape per request."""
    args = dict(name=f"decode_32k_bf16_b{batch}" + ("_exact" if exact else ""), seed=seed,
                ctx_lens=[32768] * batch, n_q=1, idx_dtype="bf16", n_heads_idx=64,
                head_dim_idx=128, topk=2048, w_dist="normal8", sfa_dtype="bf16",
                n_heads_sfa=128, sfa_std=0.5, exact=exact, device=device)
    args.update(kw)
    return make_case(**args)


def batched_fp8_lengths(seed=1003, batch=64, lo=4096, hi=131072):
    g = torch.Generator()
    g.manual_seed(int(seed) + 104729)
    return torch.randint(lo, hi + 1, (batch,), generator=g).tolist()


def batched_decode_fp8(seed=1003, wide=False, exact=False, device="cpu", batch=64, lo=4096,
                       hi=131072, **kw):
    """Batch 64, lengths uniform in [4096, 131072], fp8 e4m3 indexer K with a
    per-token scale and fp8 q with a per-head scale, Top-K 2048, bf16 sparse
    attention.  wide=False keeps the tiny decode's dims (4 x 64 indexer,
    16 SFA heads, w ~ U(0,1), N(0,1) data); wide=True uses the 32K decode's
    dims and distributions."""
    lens = batched_fp8_lengths(seed, batch, lo, hi)
    if wide:
        dims = dict(n_heads_idx=64, head_dim_idx=128, w_dist="normal8", n_heads_sfa=128, sfa_std=0.5)
    else:
        dims = dict(n_heads_idx=4, head_dim_idx=64, w_dist="uniform", n_heads_sfa=16, sfa_std=1.0)
    args = dict(name="batched_fp8_" + ("wide" if wide else "narrow") + ("_exact" if exact else ""),
                seed=seed, ctx_lens=lens, n_q=1, idx_dtype="fp8", topk=2048, sfa_dtype="bf16",
                exact=exact, device=device, **dims)
    args.update(kw)
    return make_case(**args)


def chunked_prefill(seed=1004, prefix=61440, new=4096, exact=False, device="cpu", **kw):
    """One request, ``new`` query tokens appended to a ``prefix``-token cache
    (causal), bf16 indexer 64 x 128, Top-K 2048, bf16 sparse attention 128
    heads, distributions as the 32K decode."""
    args = dict(name=f"prefill_{prefix}+{new}_bf16" + ("_exact" if exact else ""), seed=seed,
                ctx_lens=[prefix + new], n_q=new, idx_dtype="bf16", n_heads_idx=64,
                head_dim_idx=128, topk=2048, w_dist="normal8", sfa_dtype="bf16",
                n_heads_sfa=128, sfa_std=0.5, exact=exact, device=device)
    args.update(kw)
    return make_case(**args)


def spec_verify(seed=1005, batch=16, n_q=4, ctx=262144, exact=False, device="cpu", **kw):
    """Speculative-verify decode: ``batch`` requests x ``n_q`` causal query
    tokens at ``ctx`` context, fp8 indexer (64 x 128, scales as the batched
    route), Top-K 2048 per query token, bf16 sparse attention 128 heads."""
    args = dict(name=f"spec_verify_b{batch}x{n_q}_{ctx}_fp8" + ("_exact" if exact else ""),
                seed=seed, ctx_lens=[ctx] * batch, n_q=n_q, idx_dtype="fp8", n_heads_idx=64,
                head_dim_idx=128, topk=2048, w_dist="normal8", sfa_dtype="bf16",
                n_heads_sfa=128, sfa_std=0.5, exact=exact, device=device)
    args.update(kw)
    return make_case(**args)


# ---------------------------------------------------------------------------
# Host views for the oracle: raw storage as numpy (uint16 for bf16 bits,
# uint8 for fp8 codes).
# ---------------------------------------------------------------------------
def to_numpy_raw(t: Optional[torch.Tensor]):
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.int16:
        return t.numpy().view(np.uint16)
    return t.numpy()


def permute_pages(case: Case, seed: int) -> Case:
    """The same logical case with its physical pages moved to a new random
    permutation (block table rewritten to match)."""
    g = torch.Generator()
    g.manual_seed(int(seed))
    perm = torch.randperm(case.num_pages, generator=g)  # new slot of old page p is perm[p]
    dev = case.k_cache.device
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(case.num_pages)
    def move(x):
        return None if x is None else x[inv.to(dev)].contiguous()
    bt = perm.to(torch.int32)[case.block_table.long().cpu()].to(case.block_table.device)
    return dataclasses.replace(
        case, block_table=bt, decoy_pages=perm[case.decoy_pages],
        k_cache=move(case.k_cache), k_scale=move(case.k_scale), kv_cache=move(case.kv_cache))


# ---------------------------------------------------------------------------
# Cache-append inputs: new keys and the paging they go into
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class AppendCase:
    name: str
    seed: int
    q_offsets: torch.Tensor   # int32 [B+1]
    ctx_lens: torch.Tensor    # int32 [B]
    block_table: torch.Tensor  # int32 [B][max_pages]
    num_pages: int
    max_q_per_req: int
    max_ctx: int
    k_new: torch.Tensor       # float32 [T][D]


def e4m3_midpoints() -> torch.Tensor:
    """Every midpoint between neighbouring positive finite e4m3 values, and
    the fp32 values just below and above each (values on which rounding to
    nearest even decides)."""
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float()
    pos = torch.unique(vals[torch.isfinite(vals) & (vals >= 0)])
    mids = (pos[:-1] + pos[1:]) / 2
    return torch.cat([mids, torch.nextafter(mids, torch.zeros_like(mids)),
                      torch.nextafter(mids, torch.full_like(mids, 1e9))])


def append_case(seed: int, ctx_lens, n_q, head_dim: int, name: str = "append", device="cpu",
                page_size: int = PAGE_SIZE, n_decoy: int = 3) -> AppendCase:
    """New keys for requests of lengths ``ctx_lens`` whose last ``n_q`` tokens
    are new, with shuffled pages (plus decoy pages nothing maps to).  Rows are
    N(0,1) times 2^k (k uniform in -6..6), except directed rows when there are
    enough: a zero key, a key with a zero upper half, keys whose every 32-block
    holds 448 (so the fp8 scale and the MXFP8 exponents are 1 and 0) and
    otherwise e4m3 midpoints and their fp32 neighbours of both signs, and two
    keys where x / (amax / 448) in fp32 falls exactly on a midpoint that the
    exact quotient misses."""
    g = torch.Generator()
    g.manual_seed(int(seed))
    lens = torch.tensor(list(ctx_lens), dtype=torch.int32)
    nq = torch.tensor(list(n_q) if hasattr(n_q, "__len__") else [n_q] * len(lens), dtype=torch.int32)
    B = len(lens)
    qo = torch.zeros(B + 1, dtype=torch.int32)
    qo[1:] = torch.cumsum(nq, 0)
    T, D = int(qo[-1]), int(head_dim)
    ppr = [(int(L) + page_size - 1) // page_size for L in lens]
    num_pages = sum(ppr) + n_decoy
    perm = torch.randperm(num_pages, generator=g).to(torch.int32)
    bt = torch.full((B, max(ppr) + 1), int(perm[-1]), dtype=torch.int32)
    cur = 0
    for b in range(B):
        bt[b, :ppr[b]] = perm[cur:cur + ppr[b]]
        cur += ppr[b]
    x = torch.randn((T, D), generator=g) * torch.exp2(torch.randint(-6, 7, (T, 1), generator=g).float())
    mids = e4m3_midpoints()
    if T >= 8:
        x[0] = 0.0
        x[1, D // 2:] = 0.0
        for r in (2, 3):
            pick = mids[torch.randint(0, mids.numel(), (D,), generator=g)]
            sign = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0)
            x[r] = pick * sign
            x[r, ::32] = 448.0
        for r, (am, v) in ((4, (64.0592041015625, 0.6077045202255249)), (5, (54.81887435913086, 3.303816080093384))):
            x[r] = x[r].clamp(-3, 3)
            x[r, 0], x[r, 1] = am, v
    mx = int(nq.max())
    return AppendCase(name=name, seed=int(seed), q_offsets=qo.to(device), ctx_lens=lens.to(device),
                      block_table=bt.to(device), num_pages=num_pages, max_q_per_req=mx,
                      max_ctx=int(lens.max()), k_new=x.contiguous().to(device))

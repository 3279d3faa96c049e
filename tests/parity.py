"""Run seeded cases through the GPU library and the CPU oracle, and compare.

Used by the GPU tests, ``__graft_entry__.smoke()`` and the benchmark's
correctness gate.  The GPU side goes through the C ABI binding
(``lightning_indexer_top_02_amd.dsa``); the oracle side through ``oracle``.
Nothing here computes the method itself: it only moves data and compares.

Bars (written here, used everywhere):
  * Top-K index sets: bit-exact in exact mode (integer inputs); otherwise the
    sets may differ only at positions whose oracle score lies within 1e-3
    relative of the row's K-th score (the threshold band).
  * Sparse-attention outputs: max |gpu - oracle| <= 2e-2 for bf16 and fp32
    storage, computed on the GPU's own index sets so a band difference in the
    selection cannot leak into the output comparison.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle
from lightning_indexer_top_02_amd import dsa, inputs

TOPK_BAND_REL = 1e-3
# fp8 latent: bf16 output like the bf16 route (code * 2^e dequantizes to
# bf16 exactly, so the route adds no error of its own).
OUT_TOL = {"bf16": 2e-2, "f32": 2e-2, "fp8": 2e-2}
OUT_TOL_FP8_ROUTE = 6e-2


def to_device(case: inputs.Case, device="cuda") -> inputs.Case:
    def mv(x):
        return None if x is None else x.to(device)
    return dataclasses.replace(
        case, q_offsets=mv(case.q_offsets), ctx_lens=mv(case.ctx_lens), block_table=mv(case.block_table),
        q_idx=mv(case.q_idx), q_scale=mv(case.q_scale), weights=mv(case.weights), k_cache=mv(case.k_cache),
        k_scale=mv(case.k_scale), q_sfa=mv(case.q_sfa), kv_cache=mv(case.kv_cache))


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------
def paged_of(case: inputs.Case) -> dsa.Paged:
    return dsa.make_paged(case.q_offsets, case.ctx_lens, case.block_table, case.num_pages,
                          max_q_per_req=case.max_q_per_req, max_ctx_len=case.max_ctx,
                          num_q_tokens=case.num_tokens)


def indexer_of(case: inputs.Case, topk=None, flags=0) -> dsa.Indexer:
    return dsa.make_indexer(case.q_idx, case.weights, case.k_cache, topk or case.topk, case.idx_dtype,
                            q_scale=case.q_scale, k_scale=case.k_scale, flags=flags)


def indexer_routes(case: inputs.Case):
    """Flags that force each indexer route the case supports."""
    routes = {"default": 0, "positions": dsa.INDEXER_SCORE_POSITIONS}
    if case.idx_dtype != "f32" and case.n_heads_idx <= 64:
        routes["rows"] = dsa.INDEXER_SCORE_ROWS
    return routes


def sfa_tensors(case: inputs.Case):
    dt = torch.float32 if case.sfa_dtype == "f32" else torch.int16
    out = torch.empty((case.num_tokens, case.n_heads_sfa, case.v_dim), dtype=dt, device=case.q_sfa.device)
    lse = torch.empty((case.num_tokens, case.n_heads_sfa), dtype=torch.float32, device=case.q_sfa.device)
    return out, lse


def gpu_indexer_topk(case: inputs.Case, topk=None, flags=0) -> torch.Tensor:
    """Indices from dsa_indexer_topk (route chosen by the library unless flags force one)."""
    K = topk or case.topk
    out = torch.full((case.num_tokens, K), -7, dtype=torch.int32, device=case.q_idx.device)
    paged, idx = paged_of(case), indexer_of(case, K, flags)
    ws = dsa.new_workspace(dsa.indexer_topk_workspace_size(paged, idx), case.q_idx.device)
    dsa.indexer_topk(paged, idx, out, workspace=ws)
    return out


def gpu_indexer_scores(case: inputs.Case, flags=0) -> torch.Tensor:
    """Weighted scores from dsa_indexer_scores; never-written entries stay NaN."""
    sc = torch.full((case.num_tokens, case.max_ctx), float("nan"), dtype=torch.float32, device=case.q_idx.device)
    dsa.indexer_scores(paged_of(case), indexer_of(case, flags=flags), sc)
    return sc


def gpu_sparse_attn(case: inputs.Case, idx: torch.Tensor):
    out, lse = sfa_tensors(case)
    sfa = dsa.make_sfa(case.q_sfa, case.kv_cache, out, case.scale, case.sfa_dtype, lse=lse, v_dim=case.v_dim)
    dsa.sparse_attn(paged_of(case), sfa, idx.to(torch.int32).contiguous())
    return out, lse


def gpu_fused_decode(case: inputs.Case):
    out, lse = sfa_tensors(case)
    idx = torch.full((case.num_tokens, case.topk), -7, dtype=torch.int32, device=case.q_idx.device)
    sfa = dsa.make_sfa(case.q_sfa, case.kv_cache, out, case.scale, case.sfa_dtype, lse=lse, v_dim=case.v_dim)
    dsa.fused_decode(paged_of(case), indexer_of(case), sfa, topk_idx=idx)
    return idx, out, lse


def out_to_f64(out: torch.Tensor, dtype: str) -> np.ndarray:
    o = out.detach().cpu()
    if dtype in ("bf16", "fp8"):  # the fp8 latent route writes bf16
        o = o.view(torch.bfloat16)
    return o.double().numpy()


# ---------------------------------------------------------------------------
# Oracle side (host copies of the same storage)
# ---------------------------------------------------------------------------
def _np(x):
    return inputs.to_numpy_raw(x)


def oracle_indexer(case: inputs.Case, topk=None, nthreads=None):
    """(idx [T][K], scores [T][L]) from the oracle."""
    return oracle.indexer_topk(_np(case.q_offsets), _np(case.ctx_lens), _np(case.block_table),
                               case.page_size, case.idx_dtype, _np(case.q_idx), _np(case.q_scale),
                               _np(case.weights), _np(case.k_cache), _np(case.k_scale),
                               topk or case.topk, return_scores=True, nthreads=nthreads)


def oracle_sfa(case: inputs.Case, idx, nthreads=None):
    idx = idx.cpu().numpy() if isinstance(idx, torch.Tensor) else idx
    return oracle.sparse_attn(_np(case.q_offsets), _np(case.block_table), case.page_size, case.sfa_dtype,
                              case.scale, _np(case.q_sfa), _np(case.kv_cache), idx, case.v_dim,
                              nthreads=nthreads)


# ---------------------------------------------------------------------------
# Comparisons
# ---------------------------------------------------------------------------
def compare_topk(gpu_idx, ora_idx, ora_scores, vis, exact: bool, rows=None):
    """Raise AssertionError on a Top-K mismatch beyond the bar; return stats."""
    g = gpu_idx.cpu().numpy() if isinstance(gpu_idx, torch.Tensor) else np.asarray(gpu_idx)
    o = np.asarray(ora_idx)
    rows = range(o.shape[0]) if rows is None else rows
    n_diff = 0
    max_rel = 0.0
    for r, i in enumerate(rows):
        gi, oi = g[i], o[r]
        K = oi.shape[0]
        keep = min(K, int(vis[r]))
        assert np.all(gi[keep:] == -1), f"row {i}: padding {gi[keep:][:8]}"
        gs = gi[:keep]
        assert np.all(np.diff(gs) > 0), f"row {i}: not strictly ascending"
        assert gs.min(initial=0) >= 0 and gs.max(initial=0) < vis[r], f"row {i}: out of range"
        if exact:
            assert np.array_equal(gi, oi), f"row {i}: exact-mode index sets differ"
            continue
        diff = np.setxor1d(gs, oi[:keep])
        if diff.size == 0:
            continue
        s = ora_scores[r]
        tau = np.sort(s[: vis[r]])[::-1][keep - 1]
        scale = max(abs(tau), 1e-6 * np.nanmax(np.abs(s[: vis[r]])))
        rel = np.abs(s[diff] - tau) / scale
        max_rel = max(max_rel, float(rel.max()))
        assert np.all(rel <= TOPK_BAND_REL), (
            f"row {i}: {diff.size} positions differ outside the band (max rel {rel.max():.3g})")
        n_diff += diff.size
    return {"positions_in_band": n_diff, "max_rel_from_threshold": max_rel}


# Score tolerance relative to the row's term magnitude.  fp32 and bf16:
# fp32 accumulation-order differences only (bf16 products are exact in fp32).
# fp8: gfx950's fp8 MFMA does not sum its 32 products in full fp32 (an
# in-bounds probe: one 448 x 1 product plus 31 products of 2^-6 gives 448.875
# for 448.984375, and 448^2 + 31 x 1 loses 7 of the 31), so its dot products
# carry errors of a few 1e-5 of their largest product.
# MXFP8 runs on the same 16x16x128 instruction (block-scaled form).
SCORE_REL_TOL = {"f32": 1e-5, "bf16": 1e-5, "fp8": 1e-4, "mxfp8": 1e-4}


def compare_scores(gpu_scores, ora_scores, vis, exact: bool, magnitude=None, dtype="bf16"):
    """Scores of the visible positions equal (exact mode) or within
    SCORE_REL_TOL[dtype] of the row's largest term magnitude
    M_t = sum_h |w_h| ReLU(l_h) (``magnitude``: the oracle's scores with |w|;
    without it, the row's largest |score|).  The summation error of a sum of
    signed terms is bounded by the sum of their absolute values times the
    rounding unit, not by the sum itself.  Nothing past a row's position may
    be written."""
    g = gpu_scores.cpu().double().numpy() if isinstance(gpu_scores, torch.Tensor) else np.asarray(gpu_scores)
    o = np.asarray(ora_scores)
    m = np.abs(o) if magnitude is None else np.asarray(magnitude)
    worst = 0.0
    for i in range(o.shape[0]):
        v = int(vis[i])
        gi, oi = g[i, :v], o[i, :v]
        assert np.all(np.isfinite(gi)), f"row {i}: non-finite GPU score"
        assert np.all(np.isnan(g[i, v:])), f"row {i}: GPU wrote past the row's position"
        if exact:
            assert np.array_equal(gi, oi), f"row {i}: scores differ in exact mode"
            continue
        scale = float(np.max(m[i, :v], initial=0.0)) or 1.0
        err = float(np.max(np.abs(gi - oi), initial=0.0)) / scale
        assert err <= SCORE_REL_TOL[dtype], f"row {i}: score error {err:.3g} of the row's term magnitude"
        worst = max(worst, err)
    return {"score_max_rel_err": worst}


def compare_out(gpu_out, ora_out, dtype: str, tol=None, gpu_lse=None, ora_lse=None):
    g = out_to_f64(gpu_out, dtype)
    err = float(np.max(np.abs(g - ora_out))) if g.size else 0.0
    tol = OUT_TOL[dtype] if tol is None else tol
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    assert err <= tol, f"max abs output error {err:.3g} > {tol}"
    res = {"max_abs_err": err}
    if gpu_lse is not None:
        gl = gpu_lse.cpu().double().numpy()
        fin = np.isfinite(ora_lse)
        assert np.array_equal(fin, np.isfinite(gl)), "lse finiteness differs"
        lerr = float(np.max(np.abs(gl[fin] - ora_lse[fin]))) if fin.any() else 0.0
        assert lerr <= 1e-2 + 1e-3 * float(np.max(np.abs(ora_lse[fin]), initial=0)), f"lse error {lerr}"
        res["lse_max_abs_err"] = lerr
    return res


def check_case(case: inputs.Case, tol=None, nthreads=None, fused=True):
    """Full parity of one case: every indexer route (identical to each other,
    and to the oracle up to the bar), SFA on the GPU's indices, fused path."""
    vis = oracle.visible(_np(case.q_offsets), _np(case.ctx_lens))
    g_idx = gpu_indexer_topk(case)
    for name, flags in indexer_routes(case).items():
        if flags:
            assert torch.equal(g_idx, gpu_indexer_topk(case, flags=flags)), f"indexer route '{name}' disagrees"
    o_idx, o_sc = oracle_indexer(case, nthreads=nthreads)
    stats = compare_topk(g_idx, o_idx, o_sc, vis, case.exact)
    if case.sfa_dtype != "none":
        g_out, g_lse = gpu_sparse_attn(case, g_idx)
        o_out, o_lse = oracle_sfa(case, g_idx, nthreads=nthreads)
        stats.update(compare_out(g_out, o_out, case.sfa_dtype, tol, g_lse, o_lse))
        if fused:
            f_idx, f_out, f_lse = gpu_fused_decode(case)
            assert torch.equal(f_idx, g_idx), "fused decode indices differ from dsa_indexer_topk"
            assert torch.equal(f_out, g_out), "fused decode output differs from dsa_sparse_attn"
    return stats


# ---------------------------------------------------------------------------
# Large cases: check sampled query rows one by one
# ---------------------------------------------------------------------------
def rows_subcase(case: inputs.Case, rows) -> inputs.Case:
    """A host case holding only the given query rows, each as its own
    one-token request whose context is exactly that row's visible prefix, with
    the pages it touches gathered into a compact pool (data movement only)."""
    qo = case.q_offsets.cpu().numpy()
    cl = case.ctx_lens.cpu().numpy()
    bt = case.block_table.cpu().numpy()
    vis = oracle.visible(qo, cl)
    rows = [int(r) for r in rows]
    req = [int(np.searchsorted(qo, r, side="right") - 1) for r in rows]
    npg = [(int(vis[r]) + case.page_size - 1) // case.page_size for r in rows]
    used = sorted({int(p) for r, b, n in zip(rows, req, npg) for p in bt[b, :n]})
    remap = {p: k for k, p in enumerate(used)}
    new_bt = np.zeros((len(rows), max(npg)), dtype=np.int32)
    for k, (b, n) in enumerate(zip(req, npg)):
        new_bt[k, :n] = [remap[int(p)] for p in bt[b, :n]]
    sel = torch.tensor(used, dtype=torch.long, device=case.k_cache.device)
    rsel = torch.tensor(rows, dtype=torch.long, device=case.q_idx.device)

    def take(x, idx):
        return None if x is None else x[idx].cpu().contiguous()
    return dataclasses.replace(
        case, q_offsets=torch.arange(len(rows) + 1, dtype=torch.int32),
        ctx_lens=torch.tensor([int(vis[r]) for r in rows], dtype=torch.int32),
        block_table=torch.from_numpy(new_bt), num_pages=len(used), decoy_pages=torch.zeros(0, dtype=torch.long),
        q_idx=take(case.q_idx, rsel), q_scale=take(case.q_scale, rsel), weights=take(case.weights, rsel),
        k_cache=take(case.k_cache, sel), k_scale=take(case.k_scale, sel),
        q_sfa=take(case.q_sfa, rsel), kv_cache=take(case.kv_cache, sel))


def check_rows(case: inputs.Case, gpu_idx, gpu_out, rows, tol=None, nthreads=None):
    """Compare sampled rows of a large GPU result with the oracle."""
    sub = rows_subcase(case, rows)
    vis = sub.ctx_lens.numpy()
    o_idx, o_sc = oracle_indexer(sub, nthreads=nthreads)
    stats = compare_topk(gpu_idx[torch.tensor(rows, device=gpu_idx.device)].cpu(), o_idx, o_sc, vis, case.exact)
    if gpu_out is not None:
        g_idx_rows = gpu_idx[torch.tensor(rows, device=gpu_idx.device)].cpu()
        o_out, _ = oracle_sfa(sub, g_idx_rows, nthreads=nthreads)
        stats.update(compare_out(gpu_out[torch.tensor(rows, device=gpu_out.device)], o_out, case.sfa_dtype, tol))
    return stats

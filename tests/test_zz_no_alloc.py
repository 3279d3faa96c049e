"""The no-allocation fused decode (dsa_fused_decode_static) against the
workspace one (dsa_fused_decode): the same kernels, so indices, outputs and
log-sum-exps must be bit-identical.  Three calls in a row on the library's
static scratch, each smaller than the last: the scratch keeps the previous
call's contents (scores and indices where the next call's counters lie)."""
import pytest
import torch

import parity
from lightning_indexer_top_02_amd import dsa, inputs

pytestmark = pytest.mark.gpu


def _both(case):
    print(f"\n[case] static scratch {case.name} B={case.batch} T={case.num_tokens} max_ctx={case.max_ctx}",
          flush=True)
    case = parity.to_device(case)
    paged, idx = parity.paged_of(case), parity.indexer_of(case)
    res = []
    for static in (False, True):
        out, lse = parity.sfa_tensors(case)
        ii = torch.full((case.num_tokens, case.topk), -7, dtype=torch.int32, device="cuda")
        sfa = dsa.make_sfa(case.q_sfa, case.kv_cache, out, case.scale, case.sfa_dtype, lse=lse, v_dim=case.v_dim)
        if static:
            dsa.fused_decode_static(paged, idx, sfa, topk_idx=ii)
        else:
            dsa.fused_decode(paged, idx, sfa, topk_idx=ii)
        torch.cuda.synchronize()
        res.append((ii, out, lse))
    (ia, oa, la), (ib, ob, lb) = res
    assert torch.equal(ia, ib), "indices differ from dsa_fused_decode"
    assert torch.equal(oa, ob) and torch.equal(la, lb), "outputs differ from dsa_fused_decode"
    print(f"[ok] static scratch {case.name}", flush=True)
    return case


def test_static_scratch_equals_workspace_call_on_shrinking_inputs():
    # rows longer than 32768: the two-pass route (scores, histograms and
    # candidates in the scratch), 8 query rows, split sparse attention
    _both(inputs.make_case(name="static_big", seed=61, ctx_lens=[32768, 9000, 20000, 40000], n_q=[1, 1, 4, 2],
                           idx_dtype="bf16", n_heads_idx=64, head_dim_idx=128, topk=2048, sfa_dtype="bf16",
                           n_heads_sfa=128))
    # smaller: the single-launch route, whose counters and histograms now lie
    # over the previous call's scores
    _both(inputs.make_case(name="static_mid", seed=62, ctx_lens=[5000, 3000], n_q=[1, 3], idx_dtype="bf16",
                           n_heads_idx=64, head_dim_idx=128, topk=2048, sfa_dtype="bf16", n_heads_sfa=128))
    _both(inputs.make_case(name="static_small", seed=63, ctx_lens=[700], n_q=[1], idx_dtype="fp8",
                           n_heads_idx=64, head_dim_idx=128, topk=256, sfa_dtype="bf16", n_heads_sfa=64))


def test_static_scratch_matches_oracle():
    """One static-scratch call checked against the oracle directly."""
    case = parity.to_device(inputs.decode_32k(ctx_lens=[9000], exact=True, name="static_oracle"))
    paged, idx = parity.paged_of(case), parity.indexer_of(case)
    out, lse = parity.sfa_tensors(case)
    ii = torch.full((1, case.topk), -7, dtype=torch.int32, device="cuda")
    sfa = dsa.make_sfa(case.q_sfa, case.kv_cache, out, case.scale, case.sfa_dtype, lse=lse)
    dsa.fused_decode_static(paged, idx, sfa, topk_idx=ii)
    torch.cuda.synchronize()
    print(parity.check_rows(case, ii, out, [0]), flush=True)

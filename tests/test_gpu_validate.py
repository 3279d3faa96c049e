"""dsa_validate_paged on the device: each flag for data that breaks exactly
one rule of the paging contract, 0 for valid data (including unused
block-table entries holding anything).  The kernel reads only q_offsets,
ctx_lens and the used block-table entries, so the malformed inputs here are
safe; no other kernel is run on them.  The expected flags follow from the
rules themselves (no oracle: this is input validation, not the method)."""
import pytest
import torch

from lightning_indexer_top_02_amd import dsa

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(ctx=(1000, 70, 64), n_q=(1, 3, 1), num_pages=64, max_pages=16):
    """A valid three-request layout: distinct page ids, unused entries -7."""
    ctx_lens = torch.tensor(ctx, dtype=torch.int32)
    q_offsets = torch.zeros(len(ctx) + 1, dtype=torch.int32)
    q_offsets[1:] = torch.cumsum(torch.tensor(n_q, dtype=torch.int32), 0)
    bt = torch.full((len(ctx), max_pages), -7, dtype=torch.int32)
    nxt = 0
    for b, L in enumerate(ctx):
        for p in range((L + 63) // 64):
            bt[b, p] = nxt
            nxt += 1
    assert nxt <= num_pages
    return q_offsets, ctx_lens, bt, num_pages


def _validate(q_offsets, ctx_lens, bt, num_pages, **kw):
    qo, cl, b = q_offsets.to(DEV), ctx_lens.to(DEV), bt.to(DEV)
    bounds = dict(max_q_per_req=4, max_ctx_len=1024, num_q_tokens=int(q_offsets[-1]))
    bounds.update(kw)
    paged = dsa.make_paged(qo, cl, b, num_pages, **bounds)
    word = torch.full((1,), 12345, dtype=torch.int32, device=DEV)  # overwritten, not cleared
    dsa.validate_paged(paged, word)
    torch.cuda.synchronize()
    return int(word.item())


def test_valid_layout_reports_zero():
    assert _validate(*_case()) == 0


def test_unused_entries_are_not_read():
    qo, cl, bt, n = _case()
    bt[1, 5:] = 1 << 30   # request 1 uses pages 0..1 only
    assert _validate(qo, cl, bt, n) == 0


@pytest.mark.parametrize("bad", [-1, 64, 1 << 30])
def test_page_id_outside_pool(bad):
    qo, cl, bt, n = _case()
    bt[0, 15] = bad       # request 0 uses pages 0..15 (1000 positions)
    assert _validate(qo, cl, bt, n) == dsa.VALID_PAGE_ID


def test_page_id_in_last_partial_page():
    qo, cl, bt, n = _case()
    bt[1, 1] = n          # request 1: 70 positions, page 1 holds positions 64..69
    assert _validate(qo, cl, bt, n) == dsa.VALID_PAGE_ID


def test_ctx_len_above_bound():
    qo, cl, bt, n = _case()
    assert _validate(qo, cl, bt, n, max_ctx_len=999) == dsa.VALID_CTX_LEN


def test_ctx_len_below_rows():
    qo, cl, bt, n = _case(ctx=(1000, 2, 64), n_q=(1, 3, 1))
    assert _validate(qo, cl, bt, n) == dsa.VALID_CTX_LEN


def test_more_pages_than_the_row_holds():
    # 1088 positions need 17 pages; the row holds 16 (only those are read).
    # The host requires max_pages_per_req * 64 >= max_ctx_len, so a context
    # with too many pages is also longer than max_ctx_len (1024).
    qo, cl, bt, n = _case(ctx=(1000, 70, 64))
    cl[0] = 1088
    assert _validate(qo, cl, bt, n) == dsa.VALID_PAGE_COUNT | dsa.VALID_CTX_LEN


def test_rows_above_bound():
    qo, cl, bt, n = _case(n_q=(1, 3, 1))
    assert _validate(qo, cl, bt, n, max_q_per_req=2) == dsa.VALID_ROWS


@pytest.mark.parametrize("fault", ["start", "end", "decrease"])
def test_q_offsets(fault):
    qo, cl, bt, n = _case(n_q=(1, 3, 1))
    kw = {}
    if fault == "start":
        qo[0] = 1
    elif fault == "end":
        kw["num_q_tokens"] = 6
    else:
        qo[2] = 0          # request 1 ends before it starts, request 2 has 5 rows
        kw["max_q_per_req"] = 5
    assert _validate(qo, cl, bt, n, **kw) == dsa.VALID_Q_OFFSETS


def test_several_faults_are_ored():
    qo, cl, bt, n = _case()
    bt[2, 0] = -3
    assert _validate(qo, cl, bt, n, max_ctx_len=999, max_q_per_req=2) == (
        dsa.VALID_PAGE_ID | dsa.VALID_CTX_LEN | dsa.VALID_ROWS)


def test_workload_layouts_are_valid():
    """The shuffled block tables of the measured workloads meet the contract."""
    from lightning_indexer_top_02_amd import inputs
    for case in (inputs.decode_32k(batch=4, device="cpu"), inputs.spec_verify(batch=2, ctx=20000, device="cpu")):
        qo, cl, bt = case.q_offsets.cpu(), case.ctx_lens.cpu(), case.block_table.cpu()
        assert _validate(qo, cl, bt, case.num_pages, max_q_per_req=int((qo[1:] - qo[:-1]).max()),
                         max_ctx_len=case.max_ctx) == 0

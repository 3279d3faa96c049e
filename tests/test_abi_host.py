"""C ABI checks that need no GPU: the library loads, exports every function
``include/dsa.h`` declares, and rejects bad arguments on the host before any
device work (no call here passes validation, so nothing is ever launched)."""
import ctypes
import os
import re

import pytest

from lightning_indexer_top_02_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = dsa.load()
    names = declared_functions()
    assert "dsa_indexer_topk" in names and "dsa_sparse_attn" in names and "dsa_fused_decode" in names
    for n in names:
        assert hasattr(lib, n), f"libdsa.so does not export {n}"


def test_version_and_status_strings():
    assert dsa.abi_version() == 1
    for s in range(7):
        assert dsa.status_string(s) and dsa.status_string(s) != "unknown status"
    assert dsa.status_string(99) == "unknown status"


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def good_paged(**kw):
    p = dict(batch=2, num_q_tokens=5, max_q_per_req=4, max_ctx_len=1000, max_pages_per_req=16,
             page_size=64, num_pages=40, q_offsets=FAKE, ctx_lens=FAKE, block_table=FAKE)
    p.update(kw)
    return dsa.Paged(**p)


def good_indexer(**kw):
    p = dict(n_heads=64, head_dim=128, topk=256, dtype=1, q=FAKE, q_scale=None, weights=FAKE,
             k_cache=FAKE, k_scale=None, flags=0)
    p.update(kw)
    return dsa.Indexer(**p)


def good_sfa(**kw):
    p = dict(n_heads=128, qk_dim=576, v_dim=512, dtype=1, scale=1 / 24, q=FAKE, kv_cache=FAKE,
             out=FAKE, lse=None)
    p.update(kw)
    return dsa.Sfa(**p)


def call_indexer(paged, idx, out=FAKE, ws=None, ws_bytes=0):
    return dsa.load().dsa_indexer_topk(ctypes.byref(paged), ctypes.byref(idx), out, ws, ws_bytes, None)


def call_sfa(paged, sfa, idx=FAKE, topk=256, ws=None, ws_bytes=0):
    return dsa.load().dsa_sparse_attn(ctypes.byref(paged), ctypes.byref(sfa), idx, topk, ws, ws_bytes, None)


def call_fused(paged, idx, sfa, ws=None, ws_bytes=0):
    return dsa.load().dsa_fused_decode(ctypes.byref(paged), ctypes.byref(idx), ctypes.byref(sfa), None, ws,
                                       ws_bytes, None)


BAD_PAGED = [dict(batch=0), dict(num_q_tokens=0), dict(page_size=32), dict(max_pages_per_req=15),
             dict(q_offsets=None), dict(ctx_lens=None), dict(block_table=None), dict(max_q_per_req=0),
             dict(max_q_per_req=6), dict(num_pages=0), dict(num_q_tokens=1)]


@pytest.mark.parametrize("kw", BAD_PAGED, ids=[str(k) for k in BAD_PAGED])
def test_bad_paging_rejected(kw):
    assert call_indexer(good_paged(**kw), good_indexer()) == 1
    assert call_sfa(good_paged(**kw), good_sfa()) == 1
    assert call_fused(good_paged(**kw), good_indexer(), good_sfa()) == 1
    assert dsa.load().dsa_indexer_topk_workspace_size(ctypes.byref(good_paged(**kw)),
                                                      ctypes.byref(good_indexer())) == 0


BAD_INDEXER = [(dict(q=None), 1), (dict(weights=None), 1), (dict(k_cache=None), 1), (dict(topk=0), 1),
               (dict(n_heads=0), 1), (dict(dtype=7), 1), (dict(dtype=2), 1),  # fp8 without scales
               (dict(dtype=2, q_scale=FAKE), 1), (dict(n_heads=65), 2), (dict(topk=4097), 2),
               (dict(head_dim=96), 2), (dict(dtype=0, n_heads=64, head_dim=128), 2), (dict(flags=8), 1),
               (dict(flags=6), 1), (dict(flags=7), 1), (dict(dtype=0, n_heads=4, head_dim=64, flags=2), 2),
               (dict(dtype=3), 1), (dict(dtype=3, k_scale=FAKE), 1),  # MXFP8 without scales
               (dict(dtype=3, q_scale=FAKE + 2, k_scale=FAKE), 1),  # scale words misaligned
               (dict(dtype=3, q_scale=FAKE, k_scale=FAKE + 1), 1),
               (dict(dtype=3, q_scale=FAKE, k_scale=FAKE, head_dim=64), 2)]


@pytest.mark.parametrize("kw,status", BAD_INDEXER, ids=[str(k) for k, _ in BAD_INDEXER])
def test_bad_indexer_rejected(kw, status):
    assert call_indexer(good_paged(), good_indexer(**kw)) == status


def test_indexer_null_output_rejected():
    assert call_indexer(good_paged(), good_indexer(), out=None) == 1


BAD_SFA = [(dict(q=None), 1), (dict(kv_cache=None), 1), (dict(out=None), 1), (dict(dtype=3), 1),
           (dict(dtype=2, qk_dim=512), 2),
           (dict(v_dim=600), 1), (dict(scale=float("nan")), 1), (dict(qk_dim=512), 2),
           (dict(n_heads=24), 2), (dict(n_heads=144), 2)]


@pytest.mark.parametrize("kw,status", BAD_SFA, ids=[str(k) for k, _ in BAD_SFA])
def test_bad_sfa_rejected(kw, status):
    assert call_sfa(good_paged(), good_sfa(**kw)) == status


def test_sfa_topk_bounds():
    assert call_sfa(good_paged(), good_sfa(), topk=0) == 1
    assert call_sfa(good_paged(), good_sfa(), topk=5000) == 2
    assert call_sfa(good_paged(), good_sfa(), idx=None) == 1


def test_workspace_init_rejects_bad_buffers():
    lib = dsa.load()
    assert lib.dsa_workspace_init(None, 256, None) == 1
    assert lib.dsa_workspace_init(FAKE + 4, 256, None) == 1   # misaligned
    assert lib.dsa_workspace_init(FAKE, 255, None) == 1       # not whole words


def test_workspace_too_small_rejected_before_device():
    lib = dsa.load()
    p, i, s = good_paged(), good_indexer(), good_sfa()
    need = lib.dsa_indexer_topk_workspace_size(ctypes.byref(p), ctypes.byref(i))
    assert need > 0
    assert call_indexer(p, i, ws=FAKE, ws_bytes=need - 1) == 3
    assert call_indexer(p, i, ws=None, ws_bytes=need) == 3
    assert call_indexer(p, i, ws=FAKE + 8, ws_bytes=need) == 3  # misaligned
    need_f = lib.dsa_fused_decode_workspace_size(ctypes.byref(p), ctypes.byref(i), ctypes.byref(s))
    assert need_f > need
    assert call_fused(p, i, s, ws=FAKE, ws_bytes=need_f - 1) == 3


def test_workspace_sizes():
    lib = dsa.load()
    p = good_paged(num_q_tokens=5, max_ctx_len=1000)
    need = lib.dsa_indexer_topk_workspace_size(ctypes.byref(p), ctypes.byref(good_indexer()))
    # arrival counters [B] u32 | digit histograms [T][3 * 2048] u32 |
    # scores [T][round_up(L, 256)] f32, each region 256-byte aligned
    # counters | histograms | scores | selection candidates (keys, positions; min(L, 8192) per row) |
    # kept-position bitmaps (a bit per position of each 8192-position segment of the score stride)
    assert need == 256 + 5 * 6144 * 4 + 5 * 1024 * 4 + 2 * 5 * 1024 * 4 + 5 * 256 * 4
    # one row at small batch splits the index list, on both routes: fp16
    # partial outputs [splits][rows][H][512] and fp32 log-sum-exps, each
    # region 256-byte aligned (fp32: 16 splits of 16 rows for K = 256)
    one = good_paged(batch=1, num_q_tokens=1, max_q_per_req=1)
    s_bf16 = lib.dsa_sparse_attn_workspace_size(ctypes.byref(one), ctypes.byref(good_sfa()), 2048)
    assert s_bf16 > 0 and s_bf16 % 256 == 0
    s_f32 = lib.dsa_sparse_attn_workspace_size(ctypes.byref(one), ctypes.byref(good_sfa(dtype=0, n_heads=16)), 256)
    assert s_f32 == 16 * 16 * 512 * 2 + 1024


def test_indexer_scores_argument_checks():
    lib = dsa.load()
    sc = ctypes.c_void_p(FAKE)
    assert lib.dsa_indexer_scores(ctypes.byref(good_paged()), ctypes.byref(good_indexer()), None, 4096, None) == 1
    short = good_paged().max_ctx_len - 1
    assert lib.dsa_indexer_scores(ctypes.byref(good_paged()), ctypes.byref(good_indexer()), sc, short, None) == 1
    assert lib.dsa_indexer_scores(ctypes.byref(good_paged()), ctypes.byref(good_indexer(n_heads=65)), sc,
                                  1 << 20, None) == 2


def test_cache_append_argument_checks():
    lib = dsa.load()

    def call(paged=None, **kw):
        a = dict(head_dim=128, src_dtype=0, dst_dtype=2, k_new=FAKE, k_cache=FAKE, k_scale=FAKE)
        a.update(kw)
        return lib.dsa_indexer_cache_append(ctypes.byref(paged or good_paged()), ctypes.byref(dsa.CacheAppend(**a)),
                                            None)
    assert call(k_new=None) == 1 and call(k_cache=None) == 1
    assert call(k_scale=None) == 1 and call(dst_dtype=3, k_scale=None) == 1  # quantized without scales
    assert call(src_dtype=2) == 1 and call(src_dtype=3) == 1 and call(dst_dtype=4) == 1
    assert call(head_dim=96) == 2 and call(dst_dtype=3, head_dim=64) == 2
    assert call(paged=good_paged(page_size=32)) == 1 and call(paged=good_paged(batch=0)) == 1


def test_latent_append_argument_checks():
    lib = dsa.load()

    def call(paged=None, **kw):
        a = dict(qk_dim=576, v_dim=512, src_dtype=0, dst_dtype=2, x_new=FAKE, kv_cache=FAKE)
        a.update(kw)
        return lib.dsa_latent_cache_append(ctypes.byref(paged or good_paged()),
                                           ctypes.byref(dsa.LatentAppend(**a)), None)
    assert call(x_new=None) == 1 and call(kv_cache=None) == 1
    assert call(src_dtype=2) == 1 and call(dst_dtype=3) == 1 and call(dst_dtype=7) == 1
    assert call(kv_cache=FAKE + 8) == 1  # fp8 rows must be 16-byte aligned
    assert call(qk_dim=512) == 2 and call(v_dim=448) == 2
    assert call(paged=good_paged(page_size=32)) == 1 and call(paged=good_paged(batch=0)) == 1


def test_static_fused_decode_checks_before_device_work():
    """The no-allocation fused decode validates like dsa_fused_decode and
    refuses shapes whose scratch exceeds its static array, on the host."""
    lib = dsa.load()

    def call(paged, idx, sfa, out=None):
        return lib.dsa_fused_decode_static(ctypes.byref(paged), ctypes.byref(idx), ctypes.byref(sfa), out, None)
    assert call(good_paged(batch=0), good_indexer(), good_sfa()) == 1
    assert call(good_paged(), good_indexer(q=None), good_sfa()) == 1
    assert call(good_paged(), good_indexer(), good_sfa(n_heads=24)) == 2
    # 64 rows of 262144 positions: 64 MiB of scores alone
    big = good_paged(batch=64, num_q_tokens=64, max_q_per_req=1, max_ctx_len=262144, max_pages_per_req=4096)
    need = lib.dsa_fused_decode_workspace_size(ctypes.byref(big), ctypes.byref(good_indexer()), ctypes.byref(good_sfa()))
    assert need > (64 << 20)
    assert call(big, good_indexer(), good_sfa()) == 6
    assert "static" in dsa.status_string(6)


def test_validate_paged_argument_checks():
    """dsa_validate_paged refuses invalid paged arguments and a NULL or
    misaligned error word on the host, before any device work."""
    lib = dsa.load()

    def call(paged, word=FAKE):
        return lib.dsa_validate_paged(ctypes.byref(paged), word, None)
    for kw in BAD_PAGED:
        assert call(good_paged(**kw)) == 1, kw
    assert call(good_paged(), None) == 1
    assert call(good_paged(), FAKE + 2) == 1

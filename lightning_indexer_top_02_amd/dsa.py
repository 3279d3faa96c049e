"""ctypes binding of the C ABI in ``include/dsa.h`` (``libdsa.so``).

Argument marshalling only: every step of the DSA path runs in the library's
HIP kernels.  Tensors are PyTorch device tensors (PyTorch supplies device
memory and the current stream); the library never allocates.  If the built
library is missing this module raises on import of the first call, so a
missing build can never fall back to anything else.

Storage dtypes: ``"f32"`` (torch.float32), ``"bf16"`` (torch.bfloat16 or its
raw int16/uint16 bits), ``"fp8"`` (torch.float8_e4m3fn or raw uint8 codes),
``"mxfp8"`` (e4m3 codes as for fp8, with uint8 E8M0 block scales).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK = 0
INDEXER_TWO_PASS = 1  # flag: scores through the workspace instead of the fused kernel
INDEXER_SCORE_ROWS = 2  # flag: two-pass route, row-tiled MFMA scoring kernel
INDEXER_SCORE_POSITIONS = 4  # flag: two-pass route, position-tiled scoring kernel
DTYPE_CODE = {"f32": 0, "bf16": 1, "fp8": 2, "mxfp8": 3}
_STORAGE = {
    "f32": (torch.float32,),
    "bf16": (torch.bfloat16, torch.int16, torch.uint16),
    "fp8": (torch.float8_e4m3fn, torch.uint8),
    "mxfp8": (torch.float8_e4m3fn, torch.uint8),
}


class DsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class Paged(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_tokens", ctypes.c_int32),
        ("max_q_per_req", ctypes.c_int32),
        ("max_ctx_len", ctypes.c_int32),
        ("max_pages_per_req", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("q_offsets", ctypes.c_void_p),
        ("ctx_lens", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
    ]


class Indexer(ctypes.Structure):
    _fields_ = [
        ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("q_scale", ctypes.c_void_p),
        ("weights", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("flags", ctypes.c_int32),
    ]


class Sfa(ctypes.Structure):
    _fields_ = [
        ("n_heads", ctypes.c_int32),
        ("qk_dim", ctypes.c_int32),
        ("v_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p),
        ("kv_cache", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
    ]


class CacheAppend(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("src_dtype", ctypes.c_int32),
        ("dst_dtype", ctypes.c_int32),
        ("k_new", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
    ]


class LatentAppend(ctypes.Structure):
    _fields_ = [
        ("qk_dim", ctypes.c_int32),
        ("v_dim", ctypes.c_int32),
        ("src_dtype", ctypes.c_int32),
        ("dst_dtype", ctypes.c_int32),
        ("x_new", ctypes.c_void_p),
        ("kv_cache", ctypes.c_void_p),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load ``libdsa.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.c_size_t
        PP, PI, PS = ctypes.POINTER(Paged), ctypes.POINTER(Indexer), ctypes.POINTER(Sfa)
        lib.dsa_abi_version.restype = ctypes.c_int32
        lib.dsa_abi_version.argtypes = []
        lib.dsa_status_string.restype = ctypes.c_char_p
        lib.dsa_status_string.argtypes = [ctypes.c_int]
        lib.dsa_indexer_topk_workspace_size.restype = S
        lib.dsa_indexer_topk_workspace_size.argtypes = [PP, PI]
        lib.dsa_indexer_topk.restype = ctypes.c_int
        lib.dsa_indexer_topk.argtypes = [PP, PI, P, P, S, P]
        lib.dsa_indexer_scores.restype = ctypes.c_int
        lib.dsa_indexer_scores.argtypes = [PP, PI, P, ctypes.c_int64, P]
        lib.dsa_sparse_attn_workspace_size.restype = S
        lib.dsa_sparse_attn_workspace_size.argtypes = [PP, PS, ctypes.c_int32]
        lib.dsa_sparse_attn.restype = ctypes.c_int
        lib.dsa_sparse_attn.argtypes = [PP, PS, P, ctypes.c_int32, P, S, P]
        lib.dsa_fused_decode_workspace_size.restype = S
        lib.dsa_fused_decode_workspace_size.argtypes = [PP, PI, PS]
        lib.dsa_fused_decode.restype = ctypes.c_int
        lib.dsa_fused_decode.argtypes = [PP, PI, PS, P, P, S, P]
        lib.dsa_indexer_cache_append.restype = ctypes.c_int
        lib.dsa_indexer_cache_append.argtypes = [PP, ctypes.POINTER(CacheAppend), P]
        lib.dsa_latent_cache_append.restype = ctypes.c_int
        lib.dsa_latent_cache_append.argtypes = [PP, ctypes.POINTER(LatentAppend), P]
        lib.dsa_fused_decode_static.restype = ctypes.c_int
        lib.dsa_fused_decode_static.argtypes = [PP, PI, PS, P, P]
        lib.dsa_workspace_init.restype = ctypes.c_int
        lib.dsa_workspace_init.argtypes = [P, S, P]
        lib.dsa_validate_paged.restype = ctypes.c_int
        lib.dsa_validate_paged.argtypes = [PP, P, P]
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().dsa_status_string(int(status)).decode()


def abi_version() -> int:
    return int(load().dsa_abi_version())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check_tensor(t, name, dtypes, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def make_paged(q_offsets: torch.Tensor, ctx_lens: torch.Tensor, block_table: torch.Tensor,
               num_pages: int, max_q_per_req: Optional[int] = None,
               max_ctx_len: Optional[int] = None, num_q_tokens: Optional[int] = None,
               page_size: int = 64) -> Paged:
    """Paging descriptor.  The host bounds default to values read back from the
    device tensors (a synchronizing copy); pass them to avoid that."""
    for t, n in ((q_offsets, "q_offsets"), (ctx_lens, "ctx_lens"), (block_table, "block_table")):
        _check_tensor(t, n, (torch.int32,))
    B = int(ctx_lens.numel())
    if max_q_per_req is None:
        qo = q_offsets.cpu()
        max_q_per_req = int((qo[1:] - qo[:-1]).max())
    if max_ctx_len is None:
        max_ctx_len = int(ctx_lens.max().item())
    T = int(q_offsets[-1].item()) if num_q_tokens is None else int(num_q_tokens)
    return Paged(B, T, int(max_q_per_req), int(max_ctx_len), int(block_table.shape[1]), page_size,
                 int(num_pages), _ptr(q_offsets), _ptr(ctx_lens), _ptr(block_table))


def make_indexer(q, weights, k_cache, topk, dtype, q_scale=None, k_scale=None, flags=0) -> Indexer:
    _check_tensor(q, "q", _STORAGE[dtype])
    _check_tensor(k_cache, "k_cache", _STORAGE[dtype])
    _check_tensor(weights, "weights", (torch.float32,))
    scale_dtypes = (torch.uint8,) if dtype == "mxfp8" else (torch.float32,)
    _check_tensor(q_scale, "q_scale", scale_dtypes)
    _check_tensor(k_scale, "k_scale", scale_dtypes)
    T, H, D = q.shape
    if k_cache.shape[-1] != D or weights.shape != (T, H):
        raise ValueError("indexer shapes disagree")
    return Indexer(H, D, int(topk), DTYPE_CODE[dtype], _ptr(q), _ptr(q_scale), _ptr(weights),
                   _ptr(k_cache), _ptr(k_scale), int(flags))


def make_sfa(q, kv_cache, out, scale, dtype, lse=None, v_dim=512) -> Sfa:
    """dtype "fp8": bf16 q and out, kv_cache uint8 [pages][64][656] fp8
    latent rows (512 e4m3 codes, a 16-byte block of 4 E8M0 tile exponents,
    64 bf16 rope dims)."""
    io = "bf16" if dtype == "fp8" else dtype
    _check_tensor(q, "q", _STORAGE[io])
    _check_tensor(kv_cache, "kv_cache", (torch.uint8,) if dtype == "fp8" else _STORAGE[dtype])
    _check_tensor(out, "out", _STORAGE[io])
    _check_tensor(lse, "lse", (torch.float32,))
    T, H, Dqk = q.shape
    row = v_dim + 16 + 2 * (Dqk - v_dim) if dtype == "fp8" else Dqk
    if out.shape != (T, H, v_dim) or kv_cache.shape[-1] != row:
        raise ValueError("sparse-attention shapes disagree")
    return Sfa(H, Dqk, v_dim, DTYPE_CODE[dtype], float(scale), _ptr(q), _ptr(kv_cache), _ptr(out),
               _ptr(lse))


# flag bits of dsa_validate_paged
VALID_Q_OFFSETS, VALID_ROWS, VALID_CTX_LEN, VALID_PAGE_COUNT, VALID_PAGE_ID = 1, 2, 4, 8, 16


def validate_paged(paged: Paged, error_word: torch.Tensor, stream=None) -> torch.Tensor:
    """dsa_validate_paged: enqueue the device check of q_offsets, ctx_lens and
    the used block-table entries; ``error_word`` (int32 [1] on the device)
    receives the OR of the VALID_* flags, 0 when the data is valid."""
    _check_tensor(error_word, "error_word", (torch.int32,))
    if error_word.numel() < 1:
        raise ValueError("error_word needs one int32")
    st = load().dsa_validate_paged(ctypes.byref(paged), _ptr(error_word), _stream(stream))
    if st != DSA_OK:
        raise DsaError(st, "dsa_validate_paged")
    return error_word


def new_workspace(nbytes: int, device, stream=None) -> torch.Tensor:
    """Allocate a workspace and zero-fill it with dsa_workspace_init."""
    ws = torch.empty(max(int(nbytes) + 255 & ~255, 256), dtype=torch.uint8, device=device)
    workspace_init(ws, stream)
    return ws


def workspace_init(ws: torch.Tensor, stream=None):
    st = load().dsa_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if st != DSA_OK:
        raise DsaError(st, "dsa_workspace_init")


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                             f"{nbytes} needed")
        return workspace
    return new_workspace(nbytes, device)


def indexer_topk_workspace_size(paged: Paged, idx: Indexer) -> int:
    return int(load().dsa_indexer_topk_workspace_size(ctypes.byref(paged), ctypes.byref(idx)))


def indexer_topk(paged: Paged, idx: Indexer, out: torch.Tensor, workspace=None, stream=None):
    """Steps 1-2 into ``out`` (int32 [T][topk])."""
    _check_tensor(out, "out", (torch.int32,))
    lib = load()
    need = indexer_topk_workspace_size(paged, idx)
    ws = _workspace(need, out.device, workspace)
    st = lib.dsa_indexer_topk(ctypes.byref(paged), ctypes.byref(idx), _ptr(out), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream))
    if st != DSA_OK:
        raise DsaError(st, "dsa_indexer_topk")
    return out


def indexer_scores(paged: Paged, idx: Indexer, scores: torch.Tensor, stream=None):
    """Weighted indexer scores into ``scores`` (float32 [T][stride], stride >=
    max_ctx_len); entries past a row's position are left as they were."""
    _check_tensor(scores, "scores", (torch.float32,))
    if scores.dim() != 2 or scores.shape[0] < paged.num_q_tokens:
        raise ValueError("scores must be 2-D [T][stride] with a row per query token")
    st = load().dsa_indexer_scores(ctypes.byref(paged), ctypes.byref(idx), _ptr(scores),
                                   int(scores.shape[1]), _stream(stream))
    if st != DSA_OK:
        raise DsaError(st, "dsa_indexer_scores")
    return scores


def make_cache_append(k_new, src_dtype, k_cache, dst_dtype, k_scale=None) -> CacheAppend:
    _check_tensor(k_new, "k_new", _STORAGE[src_dtype])
    _check_tensor(k_cache, "k_cache", _STORAGE[dst_dtype])
    _check_tensor(k_scale, "k_scale", (torch.uint8,) if dst_dtype == "mxfp8" else (torch.float32,))
    D = k_new.shape[-1]
    if k_cache.shape[-1] != D:
        raise ValueError("k_new and k_cache dims differ")
    return CacheAppend(D, DTYPE_CODE[src_dtype], DTYPE_CODE[dst_dtype], _ptr(k_new), _ptr(k_cache), _ptr(k_scale))


def cache_append(paged: Paged, append: CacheAppend, stream=None):
    """dsa_indexer_cache_append: each request's new keys into its K-pool slots."""
    st = load().dsa_indexer_cache_append(ctypes.byref(paged), ctypes.byref(append), _stream(stream))
    if st != DSA_OK:
        raise DsaError(st, "dsa_indexer_cache_append")


def make_latent_append(x_new, src_dtype, kv_cache, dst_dtype, v_dim=512) -> LatentAppend:
    """x_new [T][576] (fp32, or bf16); kv_cache the latent pool in dst_dtype
    ("f32", "bf16", or "fp8": uint8 [pages][64][656] fp8 latent rows)."""
    _check_tensor(x_new, "x_new", _STORAGE[src_dtype])
    _check_tensor(kv_cache, "kv_cache", (torch.uint8,) if dst_dtype == "fp8" else _STORAGE[dst_dtype])
    Dqk = x_new.shape[-1]
    row = v_dim + 16 + 2 * (Dqk - v_dim) if dst_dtype == "fp8" else Dqk
    if kv_cache.shape[-1] != row:
        raise ValueError("x_new and kv_cache rows disagree")
    return LatentAppend(Dqk, v_dim, DTYPE_CODE[src_dtype], DTYPE_CODE[dst_dtype], _ptr(x_new), _ptr(kv_cache))


def latent_append(paged: Paged, append: LatentAppend, stream=None):
    """dsa_latent_cache_append: each request's new latent rows into their pool slots."""
    st = load().dsa_latent_cache_append(ctypes.byref(paged), ctypes.byref(append), _stream(stream))
    if st != DSA_OK:
        raise DsaError(st, "dsa_latent_cache_append")


def sparse_attn_workspace_size(paged: Paged, sfa: Sfa, topk: int) -> int:
    return int(load().dsa_sparse_attn_workspace_size(ctypes.byref(paged), ctypes.byref(sfa), int(topk)))


def sparse_attn(paged: Paged, sfa: Sfa, topk_idx: torch.Tensor, workspace=None, stream=None):
    """Step 3 into the ``out``/``lse`` tensors named by ``sfa``."""
    _check_tensor(topk_idx, "topk_idx", (torch.int32,))
    lib = load()
    topk = int(topk_idx.shape[-1])
    need = sparse_attn_workspace_size(paged, sfa, topk)
    ws = _workspace(need, topk_idx.device, workspace)
    st = lib.dsa_sparse_attn(ctypes.byref(paged), ctypes.byref(sfa), _ptr(topk_idx), topk, _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream))
    if st != DSA_OK:
        raise DsaError(st, "dsa_sparse_attn")


def fused_decode_workspace_size(paged: Paged, idx: Indexer, sfa: Sfa) -> int:
    return int(load().dsa_fused_decode_workspace_size(ctypes.byref(paged), ctypes.byref(idx),
                                                      ctypes.byref(sfa)))


def fused_decode(paged: Paged, idx: Indexer, sfa: Sfa, topk_idx: Optional[torch.Tensor] = None,
                 workspace=None, stream=None, device=None):
    """Steps 1-3 in one call; ``topk_idx`` (optional) receives the indices."""
    _check_tensor(topk_idx, "topk_idx", (torch.int32,))
    lib = load()
    need = fused_decode_workspace_size(paged, idx, sfa)
    dev = device if device is not None else (topk_idx.device if topk_idx is not None else "cuda")
    ws = _workspace(need, dev, workspace)
    st = lib.dsa_fused_decode(ctypes.byref(paged), ctypes.byref(idx), ctypes.byref(sfa),
                              _ptr(topk_idx), _ptr(ws), ws.numel() * ws.element_size(),
                              _stream(stream))
    if st != DSA_OK:
        raise DsaError(st, "dsa_fused_decode")


def fused_decode_static(paged: Paged, idx: Indexer, sfa: Sfa, topk_idx: Optional[torch.Tensor] = None,
                        stream=None):
    """dsa_fused_decode_static: steps 1-3 with the library's static scratch
    (no workspace, no allocation); calls on one GPU must not overlap."""
    _check_tensor(topk_idx, "topk_idx", (torch.int32,))
    st = load().dsa_fused_decode_static(ctypes.byref(paged), ctypes.byref(idx), ctypes.byref(sfa), _ptr(topk_idx),
                                        _stream(stream))
    if st != DSA_OK:
        raise DsaError(st, "dsa_fused_decode_static")

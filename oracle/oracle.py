"""ctypes marshalling for the C oracle (``dsa_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every function takes
host numpy arrays holding the raw storage of the inputs (fp32 values, bf16 bit
patterns as uint16, fp8 and MXFP8 e4m3 codes as uint8, MXFP8 E8M0 scales as
uint8) and returns fp64 results computed
by the C code; nothing numerical happens here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": 0, "bf16": 1, "fp8": 2, "mxfp8": 3}

_lib = None
_LIB_PATH = [_LIB]


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile ``dsa_oracle.c`` with gcc into ``liboracle.so`` (OpenMP, -O2)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_PATH[0] == _LIB and not os.path.exists(_LIB):
            build(force=False)
        _lib = ctypes.CDLL(_LIB_PATH[0])
        P = ctypes.c_void_p
        I = ctypes.c_int
        _lib.dsa_oracle_decode_bf16.restype = ctypes.c_double
        _lib.dsa_oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        _lib.dsa_oracle_decode_e4m3.restype = ctypes.c_double
        _lib.dsa_oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
        _lib.dsa_oracle_decode_e8m0.restype = ctypes.c_double
        _lib.dsa_oracle_decode_e8m0.argtypes = [ctypes.c_uint8]
        _lib.dsa_oracle_encode_e4m3.restype = ctypes.c_uint8
        _lib.dsa_oracle_encode_e4m3.argtypes = [ctypes.c_float]
        _lib.dsa_oracle_encode_bf16.restype = ctypes.c_uint16
        _lib.dsa_oracle_encode_bf16.argtypes = [ctypes.c_float]
        _lib.dsa_oracle_cache_append.argtypes = [I, P, P, P, I, I, I, I, P, I, P, P]
        _lib.dsa_oracle_latent_append.argtypes = [I, P, P, P, I, I, I, I, I, P, I, P]
        _lib.dsa_oracle_visible.argtypes = [I, P, P, P]
        _lib.dsa_oracle_scores.argtypes = [I, P, P, P, I, I, I, I, I, P, P, P, P, P, I, P, I]
        _lib.dsa_oracle_select.argtypes = [I, I, P, P, I, P, I]
        _lib.dsa_oracle_indexer_topk.argtypes = [I, P, P, P, I, I, I, I, I, P, P, P, P, P, I, P, I, P, I]
        _lib.dsa_oracle_sparse_attn.argtypes = [I, P, P, I, I, I, I, I, I, ctypes.c_double, P, P, P, I, P, P, I]
    return _lib


def load_library(path):
    """Load the oracle from another build of ``dsa_oracle.c`` (used by the
    test that plants mistakes in a copy of the source).  Returns the state
    that ``restore_library`` takes to switch back."""
    global _lib
    prev = _lib
    _lib = None
    real = _LIB_PATH[0]
    _LIB_PATH[0] = path
    _load()
    return prev, real


def restore_library(state):
    global _lib
    _lib, _LIB_PATH[0] = state


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _raw(a, dtype):
    want = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "mxfp8": np.uint8}[dtype]
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"{dtype} storage must be {np.dtype(want).name}, got {a.dtype}")
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def decode_bf16(bits: int) -> float:
    return _load().dsa_oracle_decode_bf16(int(bits))


def decode_e4m3(code: int) -> float:
    return _load().dsa_oracle_decode_e4m3(int(code))


def decode_e8m0(code: int) -> float:
    return _load().dsa_oracle_decode_e8m0(int(code))


def encode_e4m3(x: float) -> int:
    return int(_load().dsa_oracle_encode_e4m3(float(x)))


def encode_bf16(x: float) -> int:
    return int(_load().dsa_oracle_encode_bf16(float(x)))


def cache_append(q_offsets, ctx_lens, block_table, page_size, src_dtype, k_new, dst_dtype, k_cache,
                 k_scale=None):
    """The pools after appending k_new ([T][D] fp32, or bf16 bits as uint16)
    at positions L_b - n_b + j: returns new (k_cache, k_scale) arrays; the
    arguments are not modified."""
    q_offsets, ctx_lens, bt = _i32(q_offsets), _i32(ctx_lens), _i32(block_table)
    if bt.ndim != 2:
        raise ValueError("block_table must be [B][max_pages]")
    kn = _raw(k_new, src_dtype)
    kc = _raw(k_cache, dst_dtype).copy()
    ks = None if k_scale is None else _scales(k_scale, dst_dtype).copy()
    D = kn.shape[-1]
    if kc.shape[-1] != D:
        raise ValueError("k_new and k_cache dims differ")
    rc = _load().dsa_oracle_cache_append(len(ctx_lens), _ptr(q_offsets), _ptr(ctx_lens), _ptr(bt), bt.shape[1],
                                         int(page_size), D, DTYPES[src_dtype], _ptr(kn), DTYPES[dst_dtype],
                                         _ptr(kc), _ptr(ks))
    _check(rc, "cache_append")
    return kc, ks


def latent_append(q_offsets, ctx_lens, block_table, page_size, src_dtype, x_new, dst_dtype, kv_cache,
                  v_dim=512):
    """The latent pool after appending x_new ([T][qk_dim] fp32, or bf16 bits
    as uint16) at positions L_b - n_b + j: returns a new pool array (fp32
    [..][qk_dim], bf16 bits uint16 [..][qk_dim], or fp8 latent rows uint8
    [..][v_dim + 16 + 2 (qk_dim - v_dim)]); the arguments are not modified."""
    q_offsets, ctx_lens, bt = _i32(q_offsets), _i32(ctx_lens), _i32(block_table)
    if bt.ndim != 2:
        raise ValueError("block_table must be [B][max_pages]")
    xn = _raw(x_new, src_dtype)
    kv = _raw(kv_cache, dst_dtype).copy()
    Dqk = xn.shape[-1]
    want = v_dim + 16 + 2 * (Dqk - v_dim) if dst_dtype == "fp8" else Dqk
    if kv.shape[-1] != want:
        raise ValueError("x_new and kv_cache rows disagree")
    rc = _load().dsa_oracle_latent_append(len(ctx_lens), _ptr(q_offsets), _ptr(ctx_lens), _ptr(bt), bt.shape[1],
                                          int(page_size), Dqk, int(v_dim), DTYPES[src_dtype], _ptr(xn),
                                          DTYPES[dst_dtype], _ptr(kv))
    _check(rc, "latent_append")
    return kv


def _scales(a, dtype):
    """fp8: fp32 scales; MXFP8: E8M0 bytes (uint8); else unused."""
    if a is None:
        return None
    if dtype == "mxfp8":
        a = np.ascontiguousarray(a)
        if a.dtype != np.uint8:
            raise TypeError(f"mxfp8 scales must be uint8 E8M0 bytes, got {a.dtype}")
        return a
    return _f32(a)


def visible(q_offsets, ctx_lens) -> np.ndarray:
    q_offsets, ctx_lens = _i32(q_offsets), _i32(ctx_lens)
    B = len(ctx_lens)
    vis = np.zeros(int(q_offsets[B]), dtype=np.int32)
    _check(_load().dsa_oracle_visible(B, _ptr(q_offsets), _ptr(ctx_lens), _ptr(vis)), "visible")
    return vis


def _nthreads(nthreads):
    if nthreads is None:
        return len(os.sched_getaffinity(0))
    return int(nthreads)


def scores(q_offsets, ctx_lens, block_table, page_size, dtype, q, q_scale, w, k_cache, k_scale,
           L_out=None, nthreads=None) -> np.ndarray:
    """fp64 scores [T][L_out]; NaN where a position is not visible."""
    q_offsets, ctx_lens, block_table = _i32(q_offsets), _i32(ctx_lens), _i32(block_table)
    B = len(ctx_lens)
    T, H, D = q.shape
    if L_out is None:
        L_out = int(max(visible(q_offsets, ctx_lens).max(initial=0), 1))
    out = np.empty((T, L_out), dtype=np.float64)
    q, k_cache = _raw(q, dtype), _raw(k_cache, dtype)
    w, q_scale, k_scale = _f32(w), _scales(q_scale, dtype), _scales(k_scale, dtype)
    rc = _load().dsa_oracle_scores(B, _ptr(q_offsets), _ptr(ctx_lens), _ptr(block_table),
                                   block_table.shape[1], page_size, H, D, DTYPES[dtype],
                                   _ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_cache), _ptr(k_scale),
                                   L_out, _ptr(out), _nthreads(nthreads))
    _check(rc, "scores")
    return out


def select(score_rows, vis, K, nthreads=None) -> np.ndarray:
    score_rows = np.ascontiguousarray(score_rows, dtype=np.float64)
    vis = _i32(vis)
    T, L_out = score_rows.shape
    idx = np.empty((T, K), dtype=np.int32)
    _check(_load().dsa_oracle_select(T, L_out, _ptr(score_rows), _ptr(vis), K, _ptr(idx),
                                     _nthreads(nthreads)), "select")
    return idx


def indexer_topk(q_offsets, ctx_lens, block_table, page_size, dtype, q, q_scale, w, k_cache,
                 k_scale, K, return_scores=False, nthreads=None):
    q_offsets, ctx_lens, block_table = _i32(q_offsets), _i32(ctx_lens), _i32(block_table)
    B = len(ctx_lens)
    T, H, D = q.shape
    L_out = int(max(visible(q_offsets, ctx_lens).max(initial=0), 1))
    idx = np.empty((T, K), dtype=np.int32)
    sc = np.empty((T, L_out), dtype=np.float64) if return_scores else None
    q, k_cache = _raw(q, dtype), _raw(k_cache, dtype)
    w, q_scale, k_scale = _f32(w), _scales(q_scale, dtype), _scales(k_scale, dtype)
    rc = _load().dsa_oracle_indexer_topk(B, _ptr(q_offsets), _ptr(ctx_lens), _ptr(block_table),
                                         block_table.shape[1], page_size, H, D, DTYPES[dtype],
                                         _ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_cache),
                                         _ptr(k_scale), K, _ptr(idx), L_out, _ptr(sc),
                                         _nthreads(nthreads))
    _check(rc, "indexer_topk")
    return (idx, sc) if return_scores else idx


def sparse_attn(q_offsets, block_table, page_size, dtype, scale, q, kv_cache, idx, v_dim,
                nthreads=None):
    """Returns (out fp64 [T][H][v_dim], lse fp64 [T][H]).  dtype "fp8": bf16
    queries and fp8 latent rows as uint8 [pages][page_size][row bytes]
    (v_dim e4m3 codes, a 16-byte block of v_dim/128 E8M0 tile scales, the rope
    dims in bf16)."""
    q_offsets, block_table, idx = _i32(q_offsets), _i32(block_table), _i32(idx)
    B = len(q_offsets) - 1
    T, H, Dqk = q.shape
    K = idx.shape[1]
    out = np.empty((T, H, v_dim), dtype=np.float64)
    lse = np.empty((T, H), dtype=np.float64)
    q, kv_cache = _raw(q, "bf16" if dtype == "fp8" else dtype), _raw(kv_cache, dtype)
    if dtype == "fp8" and kv_cache.shape[-1] != v_dim + 16 + 2 * (Dqk - v_dim):
        raise ValueError("fp8 latent rows must be v_dim codes + a 16-byte E8M0 scale block + bf16 rope")
    rc = _load().dsa_oracle_sparse_attn(B, _ptr(q_offsets), _ptr(block_table), block_table.shape[1],
                                        page_size, H, Dqk, v_dim, DTYPES[dtype], float(scale),
                                        _ptr(q), _ptr(kv_cache), _ptr(idx), K, _ptr(out), _ptr(lse),
                                        _nthreads(nthreads))
    _check(rc, "sparse_attn")
    return out, lse

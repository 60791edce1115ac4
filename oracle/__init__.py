"""CPU oracle for the DSA hot path (ctypes wrapper around oracle/dsa_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with the
HIP path.  All arithmetic happens in dsa_oracle.c in double precision; this
file only converts numpy arrays to pointers.

Functions (each cites its passage in dsa_oracle.c):
  bf16_to_double, e4m3fn_to_double     exact codecs
  index_scores                         lightning-indexer scores (fp64)
  topk                                 first min(k, n) of a stable argsort of -score
  mla_attend                           sparse absorbed-MLA attention over kept rows
  mla_dense                            dense absorbed-MLA attention over all visible rows
  decode_step                          scores -> top-k -> attention for a decode batch
  e4m3fn_quantize, key_scale           fp8 encoding and the per-token key scale (float32 decisions)
  cache_append                         new tokens' keys (fp8-quantized or copied) and latent rows into caches
  mla_absorb_q, mla_absorb_out         absorbed-MLA query absorption (q_nope . W_UK) and output projection (o . W_UV)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_DT = {"f32": 0, "bf16": 1, "e4m3fn": 2}

_lib = None


class _OracleCache(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("row_stride", ctypes.c_int64),
        ("block_stride", ctypes.c_int64),
        ("scale_block_stride", ctypes.c_int64),
        ("block_table", ctypes.c_void_p),
        ("block_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("width", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # noqa: F401  (oracle/build.py)
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_bf16_to_double.restype = dbl
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3fn_to_double.restype = dbl
    lib.oracle_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_index_scores.restype = None
    lib.oracle_index_scores.argtypes = [P, i64, P, ctypes.c_int, P, P, P, P, i32, i32]
    lib.oracle_topk.restype = None
    lib.oracle_topk.argtypes = [P, P, P, i64, P, i32, i32, ctypes.c_int]
    lib.oracle_mla_attend.restype = None
    lib.oracle_mla_attend.argtypes = [P, P, P, P, ctypes.c_int, P, i32, P, i32, P, i32, i32, dbl]
    lib.oracle_mla_dense.restype = None
    lib.oracle_mla_dense.argtypes = [P, P, P, ctypes.c_int, P, i32, P, P, i32, i32, dbl]
    lib.oracle_decode_step.restype = None
    lib.oracle_decode_step.argtypes = [P, P, P, i64, P, P, ctypes.c_int, P, P, i32, P, ctypes.c_int, P, i32, i32,
                                       P, i32, i32, dbl]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    lib.oracle_e4m3fn_quantize.restype = ctypes.c_uint8
    lib.oracle_e4m3fn_quantize.argtypes = [ctypes.c_float]
    lib.oracle_key_scale.restype = ctypes.c_float
    lib.oracle_key_scale.argtypes = [P, ctypes.c_int]
    lib.oracle_mla_absorb_q.restype = None
    lib.oracle_mla_absorb_q.argtypes = [P, P, P, ctypes.c_int, P, i32, i32, i32, i32, i32]
    lib.oracle_mla_absorb_out.restype = None
    lib.oracle_mla_absorb_out.argtypes = [P, P, P, i32, i32, i32, i32]
    lib.oracle_cache_append.restype = None
    lib.oracle_cache_append.argtypes = [P, P, ctypes.c_int, P, P, ctypes.c_int, P, P, i32]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _cache_struct(cache):
    """Build the oracle's view of an inputs.Cache; returns (struct, keepalive)."""
    storage = np.ascontiguousarray(cache.storage)
    scale = None if cache.scale is None else _c(cache.scale, np.float32)
    table = None if cache.block_table is None else _c(cache.block_table, np.int32)
    st = _OracleCache(
        rows=storage.ctypes.data, scale=None if scale is None else scale.ctypes.data,
        row_stride=cache.row_stride, block_stride=cache.block_stride,
        scale_block_stride=cache.scale_block_stride,
        block_table=None if table is None else table.ctypes.data,
        block_size=cache.block_size, max_blocks=cache.max_blocks, width=cache.width, dtype=_DT[cache.dtype])
    return st, (storage, scale, table)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (timing only; the results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


def bf16_to_double(bits: int) -> float:
    return float(_load().oracle_bf16_to_double(int(bits)))


def e4m3fn_to_double(bits: int) -> float:
    return float(_load().oracle_e4m3fn_to_double(int(bits)))


def index_scores(q, q_dtype, w, keys, q_seq, q_len, ld=None) -> np.ndarray:
    """Scores [n_q, ld] float64; entries s >= q_len[i] are NaN (never written)."""
    lib = _load()
    q = np.ascontiguousarray(q)
    w = _c(w, np.float32)
    q_len = _c(q_len, np.int32)
    q_seq = None if q_seq is None else _c(q_seq, np.int32)
    n_q, H = w.shape
    if ld is None:
        ld = max(int(q_len.max()) if n_q else 1, 1)
    out = np.full((n_q, ld), np.nan, dtype=np.float64)
    st, keep = _cache_struct(keys)
    lib.oracle_index_scores(_ptr(out), ld, _ptr(q), _DT[q_dtype], _ptr(w), ctypes.byref(st), _ptr(q_seq),
                            _ptr(q_len), n_q, H)
    return out


def topk(scores, q_len, k, order="index"):
    """(indices int32 [n_q, k] padded with -1, counts int32 [n_q]) for score rows
    given as any float array (converted exactly to float64)."""
    lib = _load()
    s = _c(scores, np.float64)
    q_len = _c(q_len, np.int32)
    n_q = s.shape[0]
    idx = np.empty((n_q, k), dtype=np.int32)
    cnt = np.empty(n_q, dtype=np.int32)
    lib.oracle_topk(_ptr(idx), _ptr(cnt), _ptr(s), s.shape[1], _ptr(q_len), n_q, k, 0 if order == "index" else 1)
    return idx, cnt


def mla_attend(q, q_dtype, latent, kv_lora, indices, q_seq, softmax_scale, want_probs=False):
    """(out [n_q, H, kv_lora], lse [n_q, H], probs [n_q, H, k] or None), float64."""
    lib = _load()
    q = np.ascontiguousarray(q)
    indices = _c(indices, np.int32)
    q_seq = None if q_seq is None else _c(q_seq, np.int32)
    n_q, H = q.shape[0], q.shape[1]
    k = indices.shape[1]
    out = np.empty((n_q, H, kv_lora), dtype=np.float64)
    lse = np.empty((n_q, H), dtype=np.float64)
    probs = np.empty((n_q, H, k), dtype=np.float64) if want_probs else None
    st, keep = _cache_struct(latent)
    lib.oracle_mla_attend(_ptr(out), _ptr(lse), _ptr(probs), _ptr(q), _DT[q_dtype], ctypes.byref(st), kv_lora,
                          _ptr(indices), k, _ptr(q_seq), n_q, H, float(softmax_scale))
    return out, lse, probs


def mla_dense(q, q_dtype, latent, kv_lora, q_seq, q_len, softmax_scale):
    lib = _load()
    q = np.ascontiguousarray(q)
    q_len = _c(q_len, np.int32)
    q_seq = None if q_seq is None else _c(q_seq, np.int32)
    n_q, H = q.shape[0], q.shape[1]
    out = np.empty((n_q, H, kv_lora), dtype=np.float64)
    lse = np.empty((n_q, H), dtype=np.float64)
    st, keep = _cache_struct(latent)
    lib.oracle_mla_dense(_ptr(out), _ptr(lse), _ptr(q), _DT[q_dtype], ctypes.byref(st), kv_lora, _ptr(q_seq),
                         _ptr(q_len), n_q, H, float(softmax_scale))
    return out, lse


def decode_step(p):
    """Run one decode step of an inputs.Problem (decode=True).
    Returns dict(out, lse, scores, indices)."""
    lib = _load()
    B = p.n_q
    ld = max(p.max_len, 1)
    out = np.empty((B, p.mla_heads, p.kv_lora), dtype=np.float64)
    lse = np.empty((B, p.mla_heads), dtype=np.float64)
    scores = np.full((B, ld), np.nan, dtype=np.float64)
    idx = np.empty((B, p.topk), dtype=np.int32)
    ks, keep1 = _cache_struct(p.keys)
    ls, keep2 = _cache_struct(p.latent)
    q_idx = np.ascontiguousarray(p.q_idx)
    q_mla = np.ascontiguousarray(p.q_mla)
    w = _c(p.w_idx, np.float32)
    seq_len = _c(p.q_len, np.int32)
    lib.oracle_decode_step(_ptr(out), _ptr(lse), _ptr(scores), ld, _ptr(idx), _ptr(q_idx), _DT[p.q_idx_dtype],
                           _ptr(w), ctypes.byref(ks), p.idx_heads, _ptr(q_mla), _DT[p.q_mla_dtype], ctypes.byref(ls),
                           p.kv_lora, p.mla_heads, _ptr(seq_len), B, p.topk, float(p.softmax_scale))
    return {"out": out, "lse": lse, "scores": scores, "indices": idx}


def e4m3fn_quantize(x) -> np.ndarray:
    """uint8 e4m3fn codes of float32 values (same shape): nearest, ties to even, saturating."""
    lib = _load()
    a = _c(x, np.float32)
    flat = a.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i in range(flat.size):
        out[i] = lib.oracle_e4m3fn_quantize(ctypes.c_float(float(flat[i])))
    return out.reshape(a.shape)


def key_scale(row) -> np.float32:
    """float32 per-token scale of one key row given as float32 values."""
    r = _c(row, np.float32)
    return np.float32(_load().oracle_key_scale(_ptr(r), int(r.size)))


def _copy_cache(cache):
    import copy
    out = copy.copy(cache)
    out.storage = np.array(cache.storage, copy=True)
    if cache.scale is not None:
        out.scale = np.array(cache.scale, copy=True)
    return out


def cache_append(keys, new_keys, new_keys_dtype, latent, new_latent, seq, pos, new_latent_dtype=None):
    """Append tokens to copies of the given inputs.Cache objects (either may be
    None) and return the copies (keys, latent).  new_keys / new_latent: raw bits
    [n, width] (float32 for f32, uint16 for bf16) in new_keys_dtype /
    new_latent_dtype (default: the latent cache's dtype, bf16 for fp8 caches);
    seq (or None: all sequence 0) and pos: int32 [n]."""
    lib = _load()
    pos = _c(pos, np.int32)
    n = int(pos.shape[0])
    seq = None if seq is None else _c(seq, np.int32)
    if new_latent_dtype is None:
        new_latent_dtype = "bf16" if latent is None or latent.dtype == "e4m3fn" else latent.dtype
    k2 = None if keys is None else _copy_cache(keys)
    l2 = None if latent is None else _copy_cache(latent)
    nk = None if new_keys is None else np.ascontiguousarray(new_keys)
    nl = None if new_latent is None else np.ascontiguousarray(new_latent)
    ks = ls = None
    keep = []
    if k2 is not None:
        ks, kk = _cache_struct(k2)
        keep.append(kk)
        assert kk[0] is k2.storage and (k2.scale is None or kk[1] is k2.scale)
    if l2 is not None:
        ls, kl = _cache_struct(l2)
        keep.append(kl)
        assert kl[0] is l2.storage and (l2.scale is None or kl[1] is l2.scale)
    lib.oracle_cache_append(None if ks is None else ctypes.byref(ks), _ptr(nk), _DT[new_keys_dtype],
                            None if ls is None else ctypes.byref(ls), _ptr(nl), _DT[new_latent_dtype], _ptr(seq),
                            _ptr(pos), n)
    return k2, l2


def mla_absorb_q(q_nope, q_rope, q_dtype, w_uk):
    """float64 [n_q, H, kv_lora + rope]: q_nope [n_q, H, d_nope] and q_rope
    [n_q, H, rope] (raw bits of q_dtype, q_rope may be None), w_uk [H, d_nope,
    kv_lora] bf16 bits (uint16)."""
    lib = _load()
    q_nope = np.ascontiguousarray(q_nope)
    n_q, H, d_nope = q_nope.shape
    w_uk = _c(w_uk, np.uint16)
    kv_lora = w_uk.shape[2]
    rope = 0 if q_rope is None else q_rope.shape[2]
    q_rope = None if q_rope is None else np.ascontiguousarray(q_rope)
    out = np.empty((n_q, H, kv_lora + rope), dtype=np.float64)
    lib.oracle_mla_absorb_q(_ptr(out), _ptr(q_nope), _ptr(q_rope), _DT[q_dtype], _ptr(w_uk), n_q, H, d_nope,
                            kv_lora, rope)
    return out


def mla_absorb_out(o_lat, w_uv):
    """float64 [n_q, H, d_v]: o_lat [n_q, H, kv_lora] float32, w_uv [H, kv_lora, d_v] bf16 bits."""
    lib = _load()
    o_lat = _c(o_lat, np.float32)
    n_q, H, kv_lora = o_lat.shape
    w_uv = _c(w_uv, np.uint16)
    d_v = w_uv.shape[2]
    out = np.empty((n_q, H, d_v), dtype=np.float64)
    lib.oracle_mla_absorb_out(_ptr(out), _ptr(o_lat), _ptr(w_uv), n_q, H, kv_lora, d_v)
    return out


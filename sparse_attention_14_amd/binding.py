"""Thin ctypes binding of libdsa (include/dsa.h).

Argument marshalling only: torch tensors are passed as device pointers with the
current HIP stream; every step of the path runs in the HIP kernels.  There is
no CPU fallback: if libdsa.so is missing or a call fails, this raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DTYPES = {"f32": 0, "bf16": 1, "e4m3fn": 2}
TOPK_ORDER_INDEX = 0   # dsa_topk flags (include/dsa.h)
TOPK_ORDER_SCORE = 1
ELEM_BYTES = {"f32": 4, "bf16": 2, "e4m3fn": 1}
STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARGUMENT", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE_TOO_SMALL",
          4: "DSA_ERR_DEVICE"}


class DsaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")
        self.code = code


class DsaCache(ctypes.Structure):
    """Mirror of dsa_cache."""
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


_lib = None
EXPORTS = ("dsa_index_scores", "dsa_topk", "dsa_topk_workspace_size", "mla_sparse_attend",
           "mla_sparse_attend_workspace_size", "dsa_decode_step", "dsa_decode_step_workspace_size",
           "dsa_decode_window", "dsa_decode_window_workspace_size", "dsa_decode_shared",
           "dsa_decode_shared_workspace_size", "dsa_cache_append", "mla_absorb_q", "mla_absorb_out",
           "dsa_workspace_clear", "dsa_status_string", "dsa_decode_step_noalloc")
NOALLOC_SCRATCH_BYTES = 48 << 20   # DSA_NOALLOC_SCRATCH_BYTES


def load(path: str = LIB_PATH):
    """Load libdsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libdsa.so not found at {path}; build it with `python -m sparse_attention_14_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, i64, sz, f32, u32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float,
                                 ctypes.c_uint32)
    CP = ctypes.POINTER(DsaCache)
    sig = {
        "dsa_index_scores": (ctypes.c_int, [P, i64, P, ctypes.c_int, P, CP, P, P, i32, i32, i32, P]),
        "dsa_topk": (ctypes.c_int, [P, P, P, i64, P, i32, i32, i32, u32, P, sz, P]),
        "dsa_topk_workspace_size": (sz, [i32, i32, i32]),
        "mla_sparse_attend": (ctypes.c_int, [P, P, P, ctypes.c_int, CP, i32, P, i32, P, i32, i32, f32, P, sz, P]),
        "mla_sparse_attend_workspace_size": (sz, [i32, i32, i32, i32]),
        "dsa_decode_step": (ctypes.c_int, [P, P, P, ctypes.c_int, P, CP, i32, P, ctypes.c_int, CP, i32, i32, P, i32,
                                           i32, i32, f32, P, P, P, sz, P]),
        "dsa_decode_step_workspace_size": (sz, [i32, i32, i32, i32, i32]),
        "dsa_decode_step_noalloc": (ctypes.c_int, [P, P, P, ctypes.c_int, P, CP, i32, P, ctypes.c_int, CP, i32, i32,
                                                   P, i32, i32, i32, f32, P, P, P]),
        "dsa_decode_window": (ctypes.c_int, [P, P, P, ctypes.c_int, P, CP, i32, P, ctypes.c_int, CP, i32, i32, P,
                                             i32, i32, i32, i32, f32, P, P, P, sz, P]),
        "dsa_decode_window_workspace_size": (sz, [i32, i32, i32, i32, i32, i32]),
        "dsa_decode_shared": (ctypes.c_int, [P, P, P, ctypes.c_int, CP, i32, i32, P, i32, i32, i32, f32, P, sz, P]),
        "dsa_decode_shared_workspace_size": (sz, [i32, i32, i32, i32, i32]),
        "mla_absorb_q": (ctypes.c_int, [P, P, P, ctypes.c_int, P, i32, i32, i32, i32, i32, P]),
        "mla_absorb_out": (ctypes.c_int, [P, P, P, i32, i32, i32, i32, P]),
        "dsa_cache_append": (ctypes.c_int, [CP, P, ctypes.c_int, CP, P, ctypes.c_int, P, P, i32, P]),
        "dsa_workspace_clear": (ctypes.c_int, [P, sz, P]),
        "dsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, code: int):
    if code != 0:
        raise DsaError(fn, code)


class DeviceCache:
    """Device-resident cache plus its dsa_cache descriptor (keeps the tensors alive)."""

    def __init__(self, rows: torch.Tensor, dtype: str, width: int, block_size: int, row_stride: int,
                 block_stride: int, scale: Optional[torch.Tensor] = None, scale_block_stride: int = 0,
                 block_table: Optional[torch.Tensor] = None):
        self.rows, self.scale, self.block_table = rows, scale, block_table
        self.dtype, self.width, self.block_size = dtype, width, block_size
        self.desc = DsaCache(
            rows=rows.data_ptr(), scale=None if scale is None else scale.data_ptr(), row_stride=row_stride,
            block_stride=block_stride, scale_block_stride=scale_block_stride,
            block_table=None if block_table is None else block_table.data_ptr(), block_size=block_size,
            max_blocks=0 if block_table is None else block_table.shape[1], width=width, dtype=DTYPES[dtype])


def dsa_index_scores(scores, q, q_dtype, w, keys: DeviceCache, q_len, n_heads, max_len, q_seq=None, ld=None,
                     stream=None):
    lib = load()
    ld = scores.stride(0) if ld is None else ld
    _check("dsa_index_scores", lib.dsa_index_scores(_p(scores), ld, _p(q), DTYPES[q_dtype], _p(w),
                                                    ctypes.byref(keys.desc), _p(q_seq), _p(q_len), q_len.shape[0],
                                                    n_heads, max_len, _stream(stream)))


def dsa_topk_workspace_size(n_q, k, max_len) -> int:
    return int(load().dsa_topk_workspace_size(n_q, k, max_len))


def dsa_topk(indices, counts, scores, q_len, k, max_len, workspace=None, ld=None, flags=0, stream=None):
    lib = load()
    ld = scores.stride(0) if ld is None else ld
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_topk", lib.dsa_topk(_p(indices), _p(counts), _p(scores), ld, _p(q_len), q_len.shape[0], k, max_len,
                                    flags, _p(workspace), ws_bytes, _stream(stream)))


def mla_sparse_attend_workspace_size(n_q, n_heads, kv_lora, k) -> int:
    return int(load().mla_sparse_attend_workspace_size(n_q, n_heads, kv_lora, k))


def mla_sparse_attend(out, lse, q, q_dtype, latent: DeviceCache, kv_lora, indices, softmax_scale, q_seq=None,
                      workspace=None, stream=None):
    lib = load()
    n_q, n_heads = q.shape[0], q.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_sparse_attend", lib.mla_sparse_attend(_p(out), _p(lse), _p(q), DTYPES[q_dtype],
                                                      ctypes.byref(latent.desc), kv_lora, _p(indices),
                                                      indices.shape[1], _p(q_seq), n_q, n_heads,
                                                      float(softmax_scale), _p(workspace), ws_bytes,
                                                      _stream(stream)))


def dsa_decode_step_workspace_size(batch, max_len, k, mla_heads, kv_lora) -> int:
    return int(load().dsa_decode_step_workspace_size(batch, max_len, k, mla_heads, kv_lora))


def dsa_decode_step(out, lse, q_idx, q_idx_dtype, w_idx, keys: DeviceCache, q_mla, q_mla_dtype,
                    latent: DeviceCache, kv_lora, seq_len, max_len, k, softmax_scale, workspace, scores_out=None,
                    indices_out=None, stream=None):
    lib = load()
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("dsa_decode_step", lib.dsa_decode_step(
        _p(out), _p(lse), _p(q_idx), DTYPES[q_idx_dtype], _p(w_idx), ctypes.byref(keys.desc), q_idx.shape[1],
        _p(q_mla), DTYPES[q_mla_dtype], ctypes.byref(latent.desc), kv_lora, q_mla.shape[1], _p(seq_len),
        seq_len.shape[0], max_len, k, float(softmax_scale), _p(scores_out), _p(indices_out), _p(workspace),
        ws_bytes, _stream(stream)))


def dsa_decode_step_noalloc(out, lse, q_idx, q_idx_dtype, w_idx, keys: DeviceCache, q_mla, q_mla_dtype,
                            latent: DeviceCache, kv_lora, seq_len, max_len, k, softmax_scale, scores_out=None,
                            indices_out=None, stream=None):
    """dsa_decode_step on the library's static per-GPU scratch (no workspace, no allocation)."""
    lib = load()
    _check("dsa_decode_step_noalloc", lib.dsa_decode_step_noalloc(
        _p(out), _p(lse), _p(q_idx), DTYPES[q_idx_dtype], _p(w_idx), ctypes.byref(keys.desc), q_idx.shape[1],
        _p(q_mla), DTYPES[q_mla_dtype], ctypes.byref(latent.desc), kv_lora, q_mla.shape[1], _p(seq_len),
        seq_len.shape[0], max_len, k, float(softmax_scale), _p(scores_out), _p(indices_out), _stream(stream)))


def dsa_decode_window_workspace_size(batch, window, max_len, k, mla_heads, kv_lora) -> int:
    return int(load().dsa_decode_window_workspace_size(batch, window, max_len, k, mla_heads, kv_lora))


def dsa_decode_window(out, lse, q_idx, q_idx_dtype, w_idx, keys: DeviceCache, q_mla, q_mla_dtype,
                      latent: DeviceCache, kv_lora, seq_len, window, max_len, k, softmax_scale, workspace,
                      scores_out=None, indices_out=None, stream=None):
    """Queries are rows b * window + j of q_idx / w_idx / q_mla (see include/dsa.h)."""
    lib = load()
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("dsa_decode_window", lib.dsa_decode_window(
        _p(out), _p(lse), _p(q_idx), DTYPES[q_idx_dtype], _p(w_idx), ctypes.byref(keys.desc), q_idx.shape[1],
        _p(q_mla), DTYPES[q_mla_dtype], ctypes.byref(latent.desc), kv_lora, q_mla.shape[1], _p(seq_len),
        seq_len.shape[0], window, max_len, k, float(softmax_scale), _p(scores_out), _p(indices_out),
        _p(workspace), ws_bytes, _stream(stream)))


def dsa_decode_shared_workspace_size(batch, window, k, mla_heads, kv_lora) -> int:
    return int(load().dsa_decode_shared_workspace_size(batch, window, k, mla_heads, kv_lora))


def dsa_decode_shared(out, lse, q_mla, q_mla_dtype, latent: DeviceCache, kv_lora, indices, batch, window,
                      softmax_scale, workspace=None, stream=None):
    """Sparse attention of a layer sharing another layer's kept indices
    (rows b * window + j of q_mla / indices; see include/dsa.h)."""
    lib = load()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_decode_shared", lib.dsa_decode_shared(
        _p(out), _p(lse), _p(q_mla), DTYPES[q_mla_dtype], ctypes.byref(latent.desc), kv_lora, q_mla.shape[1],
        _p(indices), batch, window, indices.shape[1], float(softmax_scale), _p(workspace), ws_bytes,
        _stream(stream)))


def mla_absorb_q(q_out, q_nope, q_rope, w_uk, q_dtype="bf16", stream=None):
    """q_out [n_q, H, kv_lora + rope] bf16 from q_nope [n_q, H, d_nope], q_rope
    [n_q, H, rope] (or None) and w_uk [H, d_nope, kv_lora] (see include/dsa.h)."""
    lib = load()
    n_q, H, d_nope = q_nope.shape
    kv_lora = w_uk.shape[2]
    rope = 0 if q_rope is None else q_rope.shape[2]
    _check("mla_absorb_q", lib.mla_absorb_q(_p(q_out), _p(q_nope), _p(q_rope), DTYPES[q_dtype], _p(w_uk), n_q, H,
                                            d_nope, kv_lora, rope, _stream(stream)))


def mla_absorb_out(out, o_lat, w_uv, stream=None):
    """out [n_q, H, d_v] float32 from o_lat [n_q, H, kv_lora] float32 and w_uv [H, kv_lora, d_v]."""
    lib = load()
    n_q, H, kv_lora = o_lat.shape
    d_v = w_uv.shape[2]
    _check("mla_absorb_out", lib.mla_absorb_out(_p(out), _p(o_lat), _p(w_uv), n_q, H, kv_lora, d_v, _stream(stream)))


def dsa_cache_append(keys: Optional[DeviceCache], new_keys, new_keys_dtype, latent: Optional[DeviceCache],
                     new_latent, pos, seq=None, new_latent_dtype=None, stream=None):
    """Write new tokens (rows of new_keys / new_latent) at positions pos of
    sequences seq into the caches (see include/dsa.h); either cache may be None.
    new_latent_dtype defaults to the latent cache's dtype (bf16 for fp8 caches)."""
    lib = load()
    n = pos.shape[0]
    if new_latent_dtype is None:
        new_latent_dtype = "bf16" if latent is None or latent.dtype == "e4m3fn" else latent.dtype
    _check("dsa_cache_append", lib.dsa_cache_append(
        None if keys is None else ctypes.byref(keys.desc), _p(new_keys), DTYPES[new_keys_dtype],
        None if latent is None else ctypes.byref(latent.desc), _p(new_latent), DTYPES[new_latent_dtype], _p(seq),
        _p(pos), n, _stream(stream)))


def dsa_workspace_clear(workspace, stream=None):
    lib = load()
    _check("dsa_workspace_clear", lib.dsa_workspace_clear(_p(workspace), workspace.numel() * workspace.element_size(),
                                                          _stream(stream)))


def dsa_status_string(code: int) -> str:
    return load().dsa_status_string(code).decode()

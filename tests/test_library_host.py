"""CPU-side checks of libdsa: the shared library loads, exports every entry
point include/dsa.h declares, and rejects bad arguments on the host before any
HIP call (these calls never reach the device)."""
import ctypes
import os
import re

import pytest

import sparse_attention_14_amd as dsa
from sparse_attention_14_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:dsa_status|size_t|const char \*)\s*\*?\s*(\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return dsa.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(binding.EXPORTS)


def test_status_strings(lib):
    for code, text in [(0, "ok"), (1, "invalid argument"), (2, "unsupported shape or dtype"),
                       (3, "workspace too small"), (4, "device error")]:
        assert dsa.dsa_status_string(code) == text


def test_workspace_sizes_are_host_only(lib):
    assert lib.dsa_topk_workspace_size(0, 2048, 100) == 0
    assert lib.dsa_topk_workspace_size(4, 2048, 131072) > 0          # several workgroups per row
    assert lib.dsa_topk_workspace_size(2048, 2048, 65536) == 0       # one workgroup per row: no global state
    assert lib.mla_sparse_attend_workspace_size(4, 64, 512, 2048) > 0
    assert lib.mla_sparse_attend_workspace_size(2048, 64, 512, 2048) == 0
    big = lib.dsa_decode_step_workspace_size(4, 131072, 2048, 64, 512)
    assert big >= 4 * 131072 * 4


def _cache(rows=16, width=128, dtype=1, block_size=1024, row_stride=256, block_stride=256 * 1024, table=None,
           max_blocks=0, scale=None, sbs=0):
    return binding.DsaCache(rows=rows, scale=scale, row_stride=row_stride, block_stride=block_stride,
                            scale_block_stride=sbs, block_table=table, block_size=block_size, max_blocks=max_blocks,
                            width=width, dtype=dtype)


def _scores(lib, cache, q=16, q_dtype=1, w=16, n_heads=32, n_q=1, max_len=100, ld=100, scores=16, q_len=16):
    return lib.dsa_index_scores(scores, ld, q, q_dtype, w, ctypes.byref(cache), None, q_len, n_q, n_heads, max_len,
                                None)


def test_index_scores_validation(lib):
    ok = _cache()
    assert _scores(lib, ok, n_q=0) == 0                               # nothing to do
    assert _scores(lib, ok, n_q=-1) == 1
    assert _scores(lib, ok, scores=None) == 1
    assert _scores(lib, ok, q_len=None) == 1
    assert _scores(lib, ok, ld=50) == 1                               # ld < max_len
    assert _scores(lib, ok, n_heads=0) == 1
    assert _scores(lib, ok, n_heads=65) == 2
    assert _scores(lib, _cache(width=96)) == 2                        # bf16 keys need width 64 or 128
    assert _scores(lib, _cache(dtype=0, row_stride=512, block_stride=512 * 1024), q_dtype=1) == 2
    assert _scores(lib, _cache(dtype=2, row_stride=128, block_stride=128 * 1024)) == 1   # fp8 without scales
    assert _scores(lib, _cache(row_stride=200, block_stride=200 * 1024)) == 1           # row_stride < width bytes
    assert _scores(lib, _cache(rows=8)) == 2                          # misaligned rows
    assert _scores(lib, _cache(row_stride=(1 << 24) + 16, block_stride=((1 << 24) + 16) * 1024)) == 2  # > 16 MiB rows
    assert _scores(lib, _cache(table=16, max_blocks=4, block_size=48, block_stride=256 * 48)) == 2  # block % 32
    assert _scores(lib, _cache(), q_dtype=7) == 1
    assert _scores(lib, ok, n_q=65536) == 2                           # one grid row per query


def test_topk_validation(lib):
    f = lib.dsa_topk
    assert f(16, None, 16, 100, 16, 0, 2048, 100, 0, None, 0, None) == 0
    assert f(None, None, 16, 100, 16, 1, 2048, 100, 0, None, 0, None) == 1
    assert f(16, None, 16, 100, 16, 1, 0, 100, 0, None, 0, None) == 1
    assert f(16, None, 16, 100, 16, 1, 4096, 100, 0, None, 0, None) == 2      # k > 2048
    assert f(16, None, 16, 100, 16, 1, 16, 100, 2, None, 0, None) == 2        # unknown flag
    assert f(16, None, 16, 100, 16, 1, 16, 100, 7, None, 0, None) == 2
    assert f(16, None, 16, 1 << 20, 16, 1, 16, 1 << 20, 0, None, 0, None) == 2  # max_len too long
    assert f(16, None, 16, 131072, 16, 4, 2048, 131072, 0, None, 0, None) == 3  # needs a workspace
    assert f(16, None, 16, 100, 16, 65536, 2048, 100, 0, None, 0, None) == 2  # one grid row per query


def test_attend_validation(lib):
    lat = _cache(width=576, row_stride=1152, block_stride=1152 * 1024)
    f = lib.mla_sparse_attend
    args = dict(out=16, lse=None, q=16, q_dtype=1, kv_lora=512, idx=16, k=2048, n_q=1, heads=64)

    def call(**kw):
        a = dict(args, **kw)
        c = kw.get("cache", lat)
        return f(a["out"], a["lse"], a["q"], a["q_dtype"], ctypes.byref(c), a["kv_lora"], a["idx"], a["k"], None,
                 a["n_q"], a["heads"], 0.04, None, 0, None)

    assert call(n_q=0) == 0
    assert call(out=None) == 1
    assert call(k=0) == 1
    assert call(heads=24) == 2                                        # bf16 needs heads % 16 == 0
    assert call(kv_lora=448) == 2
    assert call(kv_lora=600) == 1                                     # value wider than the row
    assert call(q_dtype=0) == 2                                       # q dtype must match the cache
    assert call(k=4096) == 2
    assert call(n_q=4) == 3                                           # split plan needs a workspace
    assert call(n_q=(1 << 24) + 1) == 2
    assert call(n_q=(1 << 18), heads=64) == 2                          # n_q * heads reaches 2^24
    assert call(n_q=(1 << 20), heads=16) == 2
    assert call(q_dtype=0, kv_lora=64, n_q=(1 << 17), heads=128,
                cache=_cache(dtype=0, width=80, row_stride=320, block_stride=320 * 1024)) == 2


def test_decode_step_validation(lib):
    keys = _cache()
    lat = _cache(width=576, row_stride=1152, block_stride=1152 * 1024)
    f = lib.dsa_decode_step

    def call(batch=1, ws=None, wsb=0, k=2048, max_len=100, out=16, seq_len=16):
        return f(out, None, 16, 1, 16, ctypes.byref(keys), 32, 16, 1, ctypes.byref(lat), 512, 64, seq_len, batch,
                 max_len, k, 0.04, None, None, ws, wsb, None)

    assert call(batch=0) == 0
    assert call(out=None) == 1
    assert call(seq_len=None) == 1
    assert call(k=0) == 1
    assert call() == 3                                                # no workspace
    assert call(ws=16, wsb=64) == 3


def test_decode_window_validation(lib):
    keys = _cache()
    lat = _cache(width=576, row_stride=1152, block_stride=1152 * 1024)
    f = lib.dsa_decode_window

    def call(batch=1, window=4, ws=None, wsb=0, k=2048, max_len=100, out=16, seq_len=16):
        return f(out, None, 16, 1, 16, ctypes.byref(keys), 32, 16, 1, ctypes.byref(lat), 512, 64, seq_len, batch,
                 window, max_len, k, 0.04, None, None, ws, wsb, None)

    assert call(batch=0) == 0
    assert call(window=0) == 1
    assert call(window=-2) == 1
    assert call(window=65) == 2
    assert call(batch=16384, window=4) == 2                           # 65536 query rows
    assert call(out=None) == 1
    assert call(seq_len=None) == 1
    assert call() == 3                                                # no workspace
    assert call(ws=16, wsb=64) == 3
    # sizes: a window of w over b sequences needs at least what b * w single-token rows need
    ws1 = lib.dsa_decode_step_workspace_size(16, 131072, 2048, 64, 512)
    ws4 = lib.dsa_decode_window_workspace_size(4, 4, 131072, 2048, 64, 512)
    assert ws4 >= ws1 > 0
    assert lib.dsa_decode_window_workspace_size(4, 1, 131072, 2048, 64, 512) == \
        lib.dsa_decode_step_workspace_size(4, 131072, 2048, 64, 512)
    assert lib.dsa_decode_window_workspace_size(4, 0, 131072, 2048, 64, 512) == 0
    assert lib.dsa_decode_window_workspace_size(4, 65, 131072, 2048, 64, 512) == 0


def test_workspace_clear_validation(lib):
    assert lib.dsa_workspace_clear(None, 0, None) == 0
    assert lib.dsa_workspace_clear(None, 16, None) == 1
    assert lib.dsa_workspace_clear(16, 6, None) == 1


def test_cache_append_validation(lib):
    keys8 = _cache(dtype=2, row_stride=128, block_stride=128 * 1024, scale=16, sbs=1024)
    keys16 = _cache()
    lat = _cache(width=576, row_stride=1152, block_stride=1152 * 1024)
    f = lib.dsa_cache_append

    def call(keys=keys8, nk=16, nk_dt=1, latent=lat, nl=16, nl_dt=1, pos=16, n=4):
        return f(None if keys is None else ctypes.byref(keys), nk, nk_dt,
                 None if latent is None else ctypes.byref(latent), nl, nl_dt, None, pos, n, None)

    assert call(n=0) == 0                                             # nothing to do, no device call
    assert call(keys=None, n=0) == 0
    assert call(n=-1) == 1
    assert call(pos=None) == 1
    assert call(keys=None, latent=None) == 1
    assert call(nk=None) == 1
    assert call(nl=None) == 1
    assert call(nk_dt=7) == 1
    assert call(nl_dt=7) == 1
    assert call(nk_dt=2) == 2                                         # fp8 input for an fp8 cache
    assert call(nk=17) == 2                                           # misaligned bf16 input
    assert call(keys=keys16, nk_dt=0) == 2                            # a bf16 cache takes bf16 input only
    assert call(keys=keys16, nk=8, n=0) == 2                          # copies need 16-byte aligned input
    assert call(nl_dt=0) == 2                                         # a bf16 latent cache copies bf16 rows
    wide8 = _cache(dtype=2, width=2048, row_stride=2048, block_stride=2048 * 1024, scale=16, sbs=1024)
    assert call(keys=wide8) == 2                                      # fp8 rows up to 1024 wide
    lat8 = _cache(dtype=2, width=576, row_stride=576, block_stride=576 * 1024, scale=16, sbs=1024)
    assert call(latent=lat8, n=0) == 0                                # fp8 latent rows quantized from bf16
    assert call(latent=lat8, nl_dt=0, n=0) == 0                       # ... or from f32
    assert call(latent=lat8, nl_dt=2, n=0) == 2
    odd = _cache(width=100, row_stride=208, block_stride=208 * 1024)
    assert call(latent=odd, n=0) == 2                                 # 200-byte rows are not 16-byte chunks
    noscale = _cache(dtype=2, row_stride=128, block_stride=128 * 1024)
    assert call(keys=noscale, n=0) == 1
    assert call(n=1 << 26) == 2                                       # 64 threads per token: 2^32 work-items


def test_decode_shared_validation(lib):
    lat = _cache(width=576, row_stride=1152, block_stride=1152 * 1024)
    f = lib.dsa_decode_shared

    def call(batch=4, window=1, k=2048, out=16, idx=16, ws=None, wsb=0, heads=64, q=16):
        return f(out, None, q, 1, ctypes.byref(lat), 512, heads, idx, batch, window, k, 0.04, ws, wsb, None)

    assert call(batch=0) == 0
    assert call(batch=-1) == 1
    assert call(window=0) == 1
    assert call(window=65) == 2
    assert call(batch=(1 << 22) + 1, window=4) == 2                   # more than 2^24 queries
    assert call(batch=(1 << 16), window=4) == 2                       # 2^18 queries x 64 heads = 2^24
    assert call(out=None) == 1
    assert call(idx=None) == 1
    assert call(k=0) == 1
    assert call(k=4096) == 2
    assert call(heads=24) == 2
    assert call() == 3                                                # a 4-query step splits: needs a workspace
    need = lib.dsa_decode_shared_workspace_size(4, 1, 2048, 64, 512)
    assert need > 0 and call(ws=16, wsb=need - 1) == 3
    # the split partials of the shared step are those of mla_sparse_attend over the same queries
    assert need >= lib.mla_sparse_attend_workspace_size(4, 64, 512, 2048)
    assert lib.dsa_decode_shared_workspace_size(4, 4, 2048, 64, 512) >= \
        lib.mla_sparse_attend_workspace_size(16, 64, 512, 2048)
    assert lib.dsa_decode_shared_workspace_size(4, 0, 2048, 64, 512) == 0


def test_absorb_validation(lib):
    fq, fo = lib.mla_absorb_q, lib.mla_absorb_out

    def q(out=16, qn=16, qr=16, dt=1, w=16, n_q=4, H=64, dn=128, L=512, R=64):
        return fq(out, qn, qr, dt, w, n_q, H, dn, L, R, None)

    def o(out=16, ol=16, w=16, n_q=4, H=64, L=512, dv=128):
        return fo(out, ol, w, n_q, H, L, dv, None)

    assert q(n_q=0) == 0 and o(n_q=0) == 0
    assert q(n_q=-1) == 1 and o(n_q=-1) == 1
    assert q(out=None) == 1 and q(qn=None) == 1 and q(w=None) == 1
    assert q(qr=None) == 1                                            # rope > 0 needs its part
    assert q(qr=None, R=0, n_q=0) == 0
    assert q(dt=0) == 2                                               # bf16 only
    assert q(dt=9) == 1
    assert q(dn=100) == 2 and q(L=500) == 2 and q(R=60) == 2
    assert q(qn=24) == 2                                              # 16-byte alignment
    assert o(out=None) == 1 and o(ol=None) == 1 and o(w=None) == 1
    assert o(L=500) == 2 and o(dv=100) == 2 and o(ol=8) == 2
    assert o(H=0) == 1 and o(H=2000) == 2


def test_decode_step_noalloc_validation(lib):
    """The allocation-free step validates everything on the host before it
    looks up its device scratch: these calls never reach a device."""
    keys = _cache()
    lat = _cache(width=576, row_stride=1152, block_stride=1152 * 1024)
    f = lib.dsa_decode_step_noalloc

    def call(batch=1, k=2048, max_len=100, out=16, seq_len=16, heads=64, q_dt=1):
        return f(out, None, 16, q_dt, 16, ctypes.byref(keys), 32, 16, 1, ctypes.byref(lat), 512, heads, seq_len,
                 batch, max_len, k, 0.04, None, None, None)

    assert call(batch=0) == 0
    assert call(batch=-1) == 1
    assert call(out=None) == 1
    assert call(seq_len=None) == 1
    assert call(k=0) == 1
    assert call(k=4096) == 2
    assert call(heads=24) == 2
    assert call(q_dt=2) == 2
    # the scratch holds the 128K batch of 4 and the paged batch of 16 x 32K, not 96 x 16K
    assert lib.dsa_decode_step_workspace_size(4, 131072, 2048, 64, 512) <= binding.NOALLOC_SCRATCH_BYTES
    assert lib.dsa_decode_step_workspace_size(16, 32768, 2048, 64, 512) <= binding.NOALLOC_SCRATCH_BYTES
    assert lib.dsa_decode_step_workspace_size(96, 16384, 2048, 64, 512) > binding.NOALLOC_SCRATCH_BYTES
    assert call(batch=96, max_len=16384) == 3

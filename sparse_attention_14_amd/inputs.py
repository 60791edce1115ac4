"""Seeded synthetic inputs for the DSA hot path.

This module only draws random numbers and lays them out in memory: token caches
(contiguous or paged), queries, indexer head weights and sequence lengths.  It
holds none of the method's arithmetic (no scores, no selection, no attention),
which is why both the CPU oracle and the HIP path may take their inputs from it.

Workloads follow the decoder the pages describe ("GLM on an A100, in Vx",
section "The model": latent K/V per token, an indexer over every earlier token,
the best 2,048 kept) at the shapes of the GLM-5 DSA layer: 32 indexer heads of
width 128, 64 MLA heads over 576-wide latent rows (512 latent + 64 rope).

Random streams: numpy PCG64 seeded with SeedSequence([0xD5A, workload id, tensor
tag]), one stream per tensor, so every tensor is reproducible on its own.
Distribution notation N(mu, sigma) means standard deviation sigma.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

ELEM_BYTES = {"f32": 4, "bf16": 2, "e4m3fn": 1}

# NaN bit patterns used to poison storage that no correct read may touch.
_NAN_BITS = {"f32": 0x7FC00000, "bf16": 0x7FC0, "e4m3fn": 0x7F}

_TAGS = {
    "q_idx": 1, "w_idx": 2, "keys": 3, "key_scale": 4, "q_mla": 5, "latent": 6,
    "lens": 7, "block_perm": 8, "ties": 9, "ties_src": 10, "append_keys": 11, "append_latent": 12,
    "q_nope": 13, "q_rope": 14, "w_uk": 15, "w_uv": 16, "o_lat": 17,
}


def rng_for(workload_id: int, tag: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0xD5A, int(workload_id), _TAGS[tag]])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (torch's cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_e4m3fn_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP float8 e4m3fn bytes (uint8), round to nearest even (torch's cast).
    Values are clipped to +-448 first so the cast saturates instead of producing NaN."""
    import torch
    x = np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> raw element bits of dtype (f32 kept as float32)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "e4m3fn":
        return to_e4m3fn_bits(x)
    raise ValueError(dtype)


@dataclass
class Cache:
    """A per-token row cache in device-style storage.

    storage: uint8 [num_blocks, block_size, width * elem_bytes] (raw element bits).
    Token t of sequence b is in block (block_table[b, t // block_size] if paged,
    else b) at slot t % block_size.  scale (fp8 only): float32 [num_blocks, block_size].
    """
    storage: np.ndarray
    dtype: str
    width: int
    block_size: int
    block_table: Optional[np.ndarray] = None
    scale: Optional[np.ndarray] = None

    @property
    def num_blocks(self) -> int:
        return self.storage.shape[0]

    @property
    def row_stride(self) -> int:
        return self.width * ELEM_BYTES[self.dtype]

    @property
    def block_stride(self) -> int:
        return self.block_size * self.row_stride

    @property
    def scale_block_stride(self) -> int:
        return self.block_size

    @property
    def max_blocks(self) -> int:
        return 0 if self.block_table is None else self.block_table.shape[1]

    @property
    def paged(self) -> bool:
        return self.block_table is not None


@dataclass
class Problem:
    """Everything one pass of the hot path reads, plus the workload's constants.

    Query i belongs to sequence q_seq[i] and sees tokens 0..q_len[i]-1.
    q_idx: [n_q, idx_heads, idx_dim] raw bits (float32 for f32, uint16 for bf16);
    w_idx: float32 [n_q, idx_heads]; q_mla: [n_q, mla_heads, kv_lora + rope].
    """
    name: str
    q_idx: np.ndarray
    q_idx_dtype: str
    w_idx: np.ndarray
    keys: Cache
    q_mla: np.ndarray
    q_mla_dtype: str
    latent: Cache
    q_seq: np.ndarray
    q_len: np.ndarray
    topk: int
    kv_lora: int
    rope: int
    softmax_scale: float
    decode: bool
    meta: dict = field(default_factory=dict)

    @property
    def n_q(self) -> int:
        return int(self.q_len.shape[0])

    @property
    def idx_heads(self) -> int:
        return int(self.q_idx.shape[1])

    @property
    def idx_dim(self) -> int:
        return int(self.q_idx.shape[2])

    @property
    def mla_heads(self) -> int:
        return int(self.q_mla.shape[1])

    @property
    def max_len(self) -> int:
        return int(self.q_len.max()) if self.n_q else 0


@dataclass(frozen=True)
class Workload:
    """A named workload; every constant it needs is stated here."""
    name: str
    wid: int                       # seed id
    batch: int                     # sequences
    seq_len: tuple                 # (lo, hi) inclusive, drawn uniformly per sequence; lo == hi: fixed
    idx_heads: int
    idx_dim: int
    q_idx_dtype: str
    key_dtype: str
    q_idx_sigma: float
    key_sigma: float
    w_lo: float
    w_hi: float
    topk: int
    mla_heads: int
    kv_lora: int
    rope: int
    q_mla_dtype: str
    latent_dtype: str
    q_mla_sigma: float
    latent_sigma: float
    softmax_scale: float
    paged: bool = False
    block_size: int = 64
    key_scale_range: tuple = (0.5, 2.0)   # fp8 keys only
    tie_fraction: float = 0.0
    prefill_queries: int = 0       # > 0: one sequence, queries at the last positions (chunked prefill)
    spare_blocks: int = 2          # poisoned blocks beyond the used ones (paged)
    capacity_pad: int = 0          # poisoned rows beyond the longest sequence (contiguous)
    window: int = 1                # decode: queries per sequence, at its last `window` positions


def _fill_cache_rows(storage_rows: np.ndarray, dtype: str, rng: np.random.Generator, sigma: float,
                     count: int, width: int, chunk: int = 1 << 20) -> None:
    """Fill storage_rows (uint8 [count, width * esize]) with encoded N(0, sigma) values, chunked."""
    eb = ELEM_BYTES[dtype]
    done = 0
    rows_per_chunk = max(1, chunk // width)
    while done < count:
        m = min(rows_per_chunk, count - done)
        x = rng.standard_normal((m, width), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        bits = encode(x, dtype)
        storage_rows[done:done + m] = bits.view(np.uint8).reshape(m, width * eb)
        done += m


def _fill_quantized_rows(storage_rows: np.ndarray, rng: np.random.Generator, sigma: float, count: int, width: int,
                         chunk: int = 1 << 20) -> np.ndarray:
    """fp8 rows of N(0, sigma) values stored the way a cache writer stores them:
    per row s = max(max |x| / 448, 2^-126) in float32 and bytes = e4m3fn(x / s)
    (torch's round-to-nearest-even cast).  Returns the float32 scales [count]."""
    scales = np.empty(count, dtype=np.float32)
    done = 0
    rows_per_chunk = max(1, chunk // width)
    while done < count:
        m = min(rows_per_chunk, count - done)
        x = rng.standard_normal((m, width), dtype=np.float32) * np.float32(sigma)
        s = np.maximum(np.abs(x).max(axis=1) / np.float32(448), np.float32(2.0 ** -126)).astype(np.float32)
        storage_rows[done:done + m] = to_e4m3fn_bits((x / s[:, None]).astype(np.float32))
        scales[done:done + m] = s
        done += m
    return scales


def _poison(storage: np.ndarray, dtype: str) -> None:
    eb = ELEM_BYTES[dtype]
    pat = np.array([_NAN_BITS[dtype]], dtype={1: np.uint8, 2: np.uint16, 4: np.uint32}[eb]).view(np.uint8)
    flat = storage.reshape(-1, eb)
    flat[:] = pat


def _layout(wl: Workload, lens: np.ndarray, rng_perm: np.random.Generator):
    """Physical placement shared by the key and latent caches.

    Returns (num_blocks, block_size, block_table or None, place) where place[b]
    is a list of (block, slot0, t0, count) runs covering tokens 0..lens[b]-1."""
    B = len(lens)
    if not wl.paged:
        cap = int(lens.max()) + wl.capacity_pad if B else 1
        cap = max(cap, 1)
        place = [[(b, 0, 0, int(lens[b]))] for b in range(B)]
        return B, cap, None, place
    bs = wl.block_size
    nblk = [(int(n) + bs - 1) // bs for n in lens]
    used = int(sum(nblk))
    total = used + wl.spare_blocks
    perm = rng_perm.permutation(used).astype(np.int64)
    max_blocks = max(max(nblk) if nblk else 1, 1)
    # Unused table entries point at a spare (poisoned) block so a stray read shows NaN.
    spare = used if wl.spare_blocks > 0 else 0
    table = np.full((B, max_blocks), spare, dtype=np.int32)
    place = []
    k = 0
    for b in range(B):
        runs = []
        for j in range(nblk[b]):
            p = int(perm[k]); k += 1
            table[b, j] = p
            t0 = j * bs
            runs.append((p, 0, t0, min(bs, int(lens[b]) - t0)))
        place.append(runs)
    return total, bs, table, place


def _make_cache(wl: Workload, lens, dtype, width, sigma, tag, layout, scale_range=None) -> Cache:
    num_blocks, bs, table, place = layout
    eb = ELEM_BYTES[dtype]
    storage = np.empty((num_blocks, bs, width * eb), dtype=np.uint8)
    _poison(storage, dtype)
    scale = None
    if dtype == "e4m3fn":
        scale = np.full((num_blocks, bs), np.nan, dtype=np.float32)
    rng = rng_for(wl.wid, tag)
    rng_s = rng_for(wl.wid, "key_scale")
    # Draw values in logical token order, sequence by sequence, then place them.
    for b, runs in enumerate(place):
        n = int(lens[b])
        if n == 0:
            continue
        logical = np.empty((n, width * eb), dtype=np.uint8)
        if dtype == "e4m3fn" and scale_range is None:
            sc = _fill_quantized_rows(logical, rng, sigma, n, width)
        else:
            _fill_cache_rows(logical, dtype, rng, sigma, n, width)
            if scale is not None:
                lo, hi = scale_range
                sc = rng_s.uniform(lo, hi, size=n).astype(np.float32)
        for (p, s0, t0, cnt) in runs:
            storage[p, s0:s0 + cnt] = logical[t0:t0 + cnt]
            if scale is not None:
                scale[p, s0:s0 + cnt] = sc[t0:t0 + cnt]
    return Cache(storage=storage, dtype=dtype, width=width, block_size=bs, block_table=table, scale=scale)


def token_location(cache: Cache, seq: int, t: int):
    """(block, slot) of token t of sequence seq: plain layout bookkeeping."""
    if cache.block_table is None:
        return seq, t
    return int(cache.block_table[seq, t // cache.block_size]), t % cache.block_size


def copy_token(cache: Cache, seq: int, dst: int, src: int) -> None:
    """Make token dst an exact byte copy of token src (row and, for fp8, scale)."""
    pd, sd = token_location(cache, seq, dst)
    ps, ss = token_location(cache, seq, src)
    cache.storage[pd, sd] = cache.storage[ps, ss]
    if cache.scale is not None:
        cache.scale[pd, sd] = cache.scale[ps, ss]


def _inject_ties(wl: Workload, keys: Cache, lens: np.ndarray) -> dict:
    """Copy the key bytes (and scale) of uniformly chosen source tokens onto
    floor(tie_fraction * n) other positions per sequence, so their indexer
    scores tie exactly.  Returns {seq: (dst array, src array)}."""
    rng = rng_for(wl.wid, "ties")
    out = {}
    for b, n in enumerate(lens):
        n = int(n)
        m = int(np.floor(wl.tie_fraction * n))
        if m == 0 or n < 2:
            continue
        pos = rng.permutation(n)
        dst = np.sort(pos[:m])
        pool = pos[m:]
        src = pool[rng.integers(0, len(pool), size=m)]
        for d, s in zip(dst, src):
            copy_token(keys, b, int(d), int(s))
        out[b] = (dst.astype(np.int64), src.astype(np.int64))
    return out


def make_problem(wl: Workload) -> Problem:
    if wl.prefill_queries > 0:
        n_ctx = int(wl.seq_len[1])
        lens_seq = np.array([n_ctx], dtype=np.int64)
        nq = wl.prefill_queries
        q_len = (np.arange(n_ctx - nq, n_ctx, dtype=np.int64) + 1).astype(np.int32)
        q_seq = np.zeros(nq, dtype=np.int32)
    else:
        lo, hi = wl.seq_len
        if lo == hi:
            lens_seq = np.full(wl.batch, lo, dtype=np.int64)
        else:
            lens_seq = rng_for(wl.wid, "lens").integers(lo, hi + 1, size=wl.batch).astype(np.int64)
        # query j of sequence b sits at position len_b - window + j and sees up to it
        W = wl.window
        q_seq = np.repeat(np.arange(wl.batch, dtype=np.int32), W)
        q_len = np.maximum(np.repeat(lens_seq, W) - W + 1 + np.tile(np.arange(W), wl.batch), 0).astype(np.int32)
        nq = wl.batch * W
    layout = _layout(wl, lens_seq, rng_for(wl.wid, "block_perm"))
    keys = _make_cache(wl, lens_seq, wl.key_dtype, wl.idx_dim, wl.key_sigma, "keys", layout, wl.key_scale_range)
    latent = _make_cache(wl, lens_seq, wl.latent_dtype, wl.kv_lora + wl.rope, wl.latent_sigma, "latent", layout)
    ties = _inject_ties(wl, keys, lens_seq) if wl.tie_fraction > 0 else {}

    r = rng_for(wl.wid, "q_idx")
    q_idx = encode(r.standard_normal((nq, wl.idx_heads, wl.idx_dim), dtype=np.float32) * np.float32(wl.q_idx_sigma),
                   wl.q_idx_dtype)
    w_idx = rng_for(wl.wid, "w_idx").uniform(wl.w_lo, wl.w_hi, size=(nq, wl.idx_heads)).astype(np.float32)
    W = wl.kv_lora + wl.rope
    r = rng_for(wl.wid, "q_mla")
    q_mla = encode(r.standard_normal((nq, wl.mla_heads, W), dtype=np.float32) * np.float32(wl.q_mla_sigma),
                   wl.q_mla_dtype)
    return Problem(name=wl.name, q_idx=q_idx, q_idx_dtype=wl.q_idx_dtype, w_idx=w_idx, keys=keys,
                   q_mla=q_mla, q_mla_dtype=wl.q_mla_dtype, latent=latent, q_seq=q_seq, q_len=q_len,
                   topk=wl.topk, kv_lora=wl.kv_lora, rope=wl.rope, softmax_scale=wl.softmax_scale,
                   decode=wl.prefill_queries == 0, meta={"ties": ties, "seq_lens": lens_seq, "workload": wl})


_S32 = float(np.float32(1.0 / np.sqrt(32.0)))

# The five workloads at their full sizes.
TINY_FP32 = Workload(
    name="tiny_fp32_decode_1k", wid=0, batch=1, seq_len=(1024, 1024), idx_heads=4, idx_dim=32,
    q_idx_dtype="f32", key_dtype="f32", q_idx_sigma=1.0, key_sigma=1.0, w_lo=0.0, w_hi=1.0, topk=256,
    mla_heads=8, kv_lora=64, rope=16, q_mla_dtype="f32", latent_dtype="f32",
    q_mla_sigma=float(1.0 / np.sqrt(80.0)), latent_sigma=float(1.0 / np.sqrt(80.0)),
    softmax_scale=float(1.0 / np.sqrt(80.0)))

DECODE_8K = Workload(
    name="glm5_decode_8k", wid=1, batch=1, seq_len=(8192, 8192), idx_heads=32, idx_dim=128,
    q_idx_dtype="bf16", key_dtype="bf16", q_idx_sigma=1.0, key_sigma=1.0, w_lo=0.0, w_hi=_S32, topk=2048,
    mla_heads=64, kv_lora=512, rope=64, q_mla_dtype="bf16", latent_dtype="bf16", q_mla_sigma=1.0,
    latent_sigma=0.05, softmax_scale=float(1.0 / np.sqrt(576.0)))

PAGED_DECODE = dataclasses.replace(DECODE_8K, name="paged_decode_16x16k_32k", wid=2, batch=16,
                                   seq_len=(16384, 32768), paged=True)

DECODE_128K_FP8 = dataclasses.replace(DECODE_8K, name="decode_128k_fp8", wid=3, batch=4,
                                      seq_len=(131072, 131072), key_dtype="e4m3fn", tie_fraction=0.01)

PREFILL_64K = dataclasses.replace(DECODE_8K, name="prefill_chunk_2048_at_64k", wid=4, batch=1,
                                  seq_len=(65536, 65536), prefill_queries=2048)

# Multi-token decode window: the known token and three guesses per sequence.
DECODE_128K_FP8_W4 = dataclasses.replace(DECODE_128K_FP8, name="decode_128k_fp8_window4", wid=5, window=4)
PAGED_DECODE_W4 = dataclasses.replace(PAGED_DECODE, name="paged_decode_16x16k_32k_window4", wid=6, window=4)

# fp8 latent rows (e4m3fn with a float32 scale per token, as the cache append
# writes them): the memory-halving variant of the 128K batch
DECODE_128K_FP8_LAT8 = dataclasses.replace(DECODE_128K_FP8, name="decode_128k_fp8_latent8", wid=7,
                                           latent_dtype="e4m3fn")

FULL_WORKLOADS = {w.name: w for w in (TINY_FP32, DECODE_8K, PAGED_DECODE, DECODE_128K_FP8, PREFILL_64K)}
WINDOW_WORKLOADS = {w.name: w for w in (DECODE_128K_FP8_W4, PAGED_DECODE_W4)}


def small(wl: Workload, **kw) -> Workload:
    """The same workload at a size the oracle finishes in seconds."""
    return dataclasses.replace(wl, **kw)


def cache_from_values(values, dtype: str, scale=None, paged_block: int = 0, seed: int = 0,
                      capacity_pad: int = 0) -> Cache:
    """Lay out explicit per-token values as a cache.

    values: float array [B, n, width] (encoded to dtype) or already-encoded raw
    bits (uint8/uint16/float32 matching dtype).  scale: [B, n] float32 (fp8).
    paged_block > 0 scatters the blocks over a random permutation (seeded)."""
    v = np.asarray(values)
    B, n, width = v.shape
    eb = ELEM_BYTES[dtype]
    raw_types = {"f32": np.float32, "bf16": np.uint16, "e4m3fn": np.uint8}
    bits = v if v.dtype == raw_types[dtype] else encode(v.astype(np.float32), dtype)
    bits = np.ascontiguousarray(bits).view(np.uint8).reshape(B, n, width * eb)
    if paged_block <= 0:
        cap = max(n + capacity_pad, 1)
        storage = np.empty((B, cap, width * eb), dtype=np.uint8)
        _poison(storage, dtype)
        storage[:, :n] = bits
        sc = None
        if dtype == "e4m3fn":
            sc = np.full((B, cap), np.nan, dtype=np.float32)
            sc[:, :n] = np.asarray(scale, dtype=np.float32)
        return Cache(storage=storage, dtype=dtype, width=width, block_size=cap, scale=sc)
    bs = paged_block
    nblk = (n + bs - 1) // bs
    used = B * nblk
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(used)
    storage = np.empty((used + 1, bs, width * eb), dtype=np.uint8)
    _poison(storage, dtype)
    sc = np.full((used + 1, bs), np.nan, dtype=np.float32) if dtype == "e4m3fn" else None
    table = np.full((B, max(nblk, 1)), used, dtype=np.int32)
    k = 0
    for b in range(B):
        for j in range(nblk):
            p = int(perm[k]); k += 1
            table[b, j] = p
            t0, t1 = j * bs, min(n, (j + 1) * bs)
            storage[p, :t1 - t0] = bits[b, t0:t1]
            if sc is not None:
                sc[p, :t1 - t0] = np.asarray(scale, dtype=np.float32)[b, t0:t1]
    return Cache(storage=storage, dtype=dtype, width=width, block_size=bs, block_table=table, scale=sc)


def append_tokens(p: Problem, window: int = 1, key_dtype: str = "bf16"):
    """New tokens to write into a decode problem's caches at the last `window`
    positions of each sequence (positions below 0 skipped).

    Returns (new_keys, new_latent, seq, pos): new_keys [n, idx_dim] raw bits in
    key_dtype ("bf16" -> uint16, "f32" -> float32) drawn N(0, key_sigma);
    new_latent [n, kv_lora + rope] raw bits in the latent dtype (bf16 for an
    fp8 latent cache) drawn N(0, latent_sigma); seq, pos int32 [n]."""
    wl = p.meta["workload"]
    lens = np.asarray(p.meta["seq_lens"], dtype=np.int64)
    seq, pos = [], []
    for b, n in enumerate(lens):
        for j in range(window):
            t = int(n) - window + j
            if t >= 0:
                seq.append(b)
                pos.append(t)
    m = len(pos)
    wid = wl.wid * 1000 + window
    nk = rng_for(wid, "append_keys").standard_normal((m, wl.idx_dim), dtype=np.float32) * np.float32(wl.key_sigma)
    W = wl.kv_lora + wl.rope
    nl = rng_for(wid, "append_latent").standard_normal((m, W), dtype=np.float32) * np.float32(wl.latent_sigma)
    latent_in = "bf16" if wl.latent_dtype == "e4m3fn" else wl.latent_dtype   # fp8 caches quantize bf16 rows
    return (encode(nk, key_dtype), encode(nl, latent_in), np.array(seq, dtype=np.int32),
            np.array(pos, dtype=np.int32))


@dataclass(frozen=True)
class AbsorbWorkload:
    """Shapes of the absorbed-MLA projections around the attention.  The pages
    give kv_lora 512 + rope 64 and 64 heads but not the per-head no-rope and
    value widths; 128 each is taken (kv_lora = 4 x 128)."""
    name: str
    wid: int
    n_q: int
    heads: int = 64
    d_nope: int = 128
    kv_lora: int = 512
    rope: int = 64
    d_v: int = 128


def make_absorb(aw: AbsorbWorkload) -> dict:
    """Seeded inputs: q_nope, q_rope ~ N(0, 1) bf16 bits; w_uk [H, d_nope, kv_lora]
    ~ N(0, 1/sqrt(d_nope)) and w_uv [H, kv_lora, d_v] ~ N(0, 1/sqrt(kv_lora)) bf16
    bits (random initialisation); o_lat [n_q, H, kv_lora] ~ N(0, 0.01) float32
    (the attention output, a weighted mean of N(0, 0.05) latent rows)."""
    H = aw.heads
    f32 = np.float32

    def normal(tag, shape, sigma):
        return rng_for(aw.wid, tag).standard_normal(shape, dtype=f32) * f32(sigma)

    return {
        "q_nope": encode(normal("q_nope", (aw.n_q, H, aw.d_nope), 1.0), "bf16"),
        "q_rope": encode(normal("q_rope", (aw.n_q, H, aw.rope), 1.0), "bf16") if aw.rope else None,
        "w_uk": encode(normal("w_uk", (H, aw.d_nope, aw.kv_lora), 1.0 / np.sqrt(aw.d_nope)), "bf16"),
        "w_uv": encode(normal("w_uv", (H, aw.kv_lora, aw.d_v), 1.0 / np.sqrt(aw.kv_lora)), "bf16"),
        "o_lat": normal("o_lat", (aw.n_q, H, aw.kv_lora), 0.01),
    }


ABSORB_DECODE = AbsorbWorkload(name="absorb_decode_4q", wid=20, n_q=4)
ABSORB_PREFILL = AbsorbWorkload(name="absorb_prefill_2048q", wid=21, n_q=2048)

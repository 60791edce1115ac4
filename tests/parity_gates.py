"""Parity gates between a computed result and the oracle (CPU only: numpy and
torch's CPU dtype casts).  The GPU tests apply them to the library's outputs;
the CPU tests apply them to deliberately wrong variants of the oracle's own
results, to show that the gates catch plausible kernel mistakes.

Scores.  Every product q_hd * khat_d reaches the accumulator exactly (bf16
times bf16, or bf16 times an e4m3fn byte decoded exactly to bf16, or an fp32
fused multiply-add), so the only error of an fp32-accumulated score is
rounding in the sums: the D-term dot product of each head, the multiply by
the head weight, the H-term head sum and, for fp8 keys, the multiply by the
token's scale.  The classical bound for such a computation is
gamma_n * cond with n = D + H + 2 terms, gamma_n = n u / (1 - n u), u = 2^-24,
and cond = sum_h |w_h| sum_d |q_hd khat_d|.  The gate allows twice that
(n = D + H + 4, factor 2, in case the matrix core's internal additions
truncate instead of rounding to nearest):

    |gpu - oracle| <= 2 (D + H + 4) 2^-24 * cond             (accumulation)

and, as the plain reading of "relative error <= tol" (2e-3 for bf16 / fp8
inputs, 1e-5 for fp32 inputs) with the accumulation bound as its floor for
scores that cancel to near zero,

    |gpu - oracle| <= tol * |oracle| + 2 (D + H + 4) 2^-24 * cond.

An oracle score of exactly 0 (every head's dot product <= 0) must be exactly 0.

Attention: per (query, head) ||gpu_o - oracle_o||_2 <= tol ||oracle_o||_2 and
|gpu_lse - oracle_lse| <= tol max(1, |oracle_lse|).

Indices: bit-exact against the oracle's top-k of the GPU's own scores; against
the oracle's own end-to-end chain, every token kept by one side only must
score within the accumulation bound of the row's k-th oracle score.
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-5, "bf16": 2e-3, "e4m3fn": 2e-3}
U32 = 2.0 ** -24


def accumulation_gamma(idx_dim: int, idx_heads: int) -> float:
    """Allowed score error per unit of condition (see the module docstring)."""
    return 2.0 * (idx_dim + idx_heads + 4) * U32


def decode_values(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw element bits -> float64 via torch's dtype casts."""
    import torch
    if dtype == "f32":
        return bits.view(np.float32).astype(np.float64)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def logical_rows(cache, seq: int, n: int) -> np.ndarray:
    """Decoded rows of tokens 0..n-1 of a sequence (float64 [n, width]), scale applied."""
    from sparse_attention_14_amd import inputs
    eb = inputs.ELEM_BYTES[cache.dtype]
    t = np.arange(n)
    if cache.block_table is None:
        blk = np.full(n, seq)
        slot = t
    else:
        blk = cache.block_table[seq, t // cache.block_size]
        slot = t % cache.block_size
    raw = cache.storage[blk, slot]                       # [n, width * eb] uint8
    elem = {1: np.uint8, 2: np.uint16, 4: np.uint32}[eb]
    vals = decode_values(np.ascontiguousarray(raw).view(elem).reshape(n, cache.width), cache.dtype)
    if cache.scale is not None:
        vals = vals * cache.scale[blk, slot].astype(np.float64)[:, None]
    return vals


def score_condition(p, i: int, memo: dict | None = None) -> np.ndarray:
    """sum_h |w_h| sum_d |q_hd khat_d| for every token of query i.  memo (optional)
    keeps each sequence's decoded |key| rows between calls."""
    n = int(p.q_len[i])
    if n == 0:
        return np.zeros(0)
    seq = int(p.q_seq[i])
    if memo is not None:
        k = memo.get(seq)
        if k is None or k.shape[0] < n:
            most = int(max(int(p.q_len[j]) for j in range(p.n_q) if int(p.q_seq[j]) == seq))
            k = memo[seq] = np.abs(logical_rows(p.keys, seq, most))
        k = k[:n]
    else:
        k = np.abs(logical_rows(p.keys, seq, n))
    q = np.abs(decode_values(p.q_idx[i].reshape(-1), p.q_idx_dtype).reshape(p.idx_heads, p.idx_dim))
    return np.abs(p.w_idx[i].astype(np.float64)) @ (q @ k.T)


class GateFailure(AssertionError):
    pass


def check_scores(p, gpu: np.ndarray, ref: np.ndarray, rows=None, tol=None, conds=None) -> dict:
    """Apply the score gates to rows of `gpu` (float32 or float64, [len(rows), >= n])
    against the oracle's `ref`.  Raises GateFailure on the first failing row.
    Returns the worst error per unit of condition, the worst plain relative
    error over all nonzero scores and over the upper half of each row's
    nonzero scores (by magnitude), and the number of scores checked."""
    tol = TOL[p.keys.dtype] if tol is None else tol
    gamma = accumulation_gamma(p.idx_dim, p.idx_heads)
    rows = range(p.n_q) if rows is None else rows
    worst_cond = 0.0
    worst_rel = 0.0
    worst_rel_upper = 0.0
    checked = 0
    memo = {}
    for r, i in enumerate(rows):
        n = int(p.q_len[i])
        if n == 0:
            continue
        g = gpu[r, :n].astype(np.float64)
        o = ref[r, :n]
        cond = score_condition(p, i, memo) if conds is None else conds[r]
        err = np.abs(g - o)
        floor = gamma * cond
        bad = err > floor
        if bad.any():
            j = int(np.argmax(np.where(bad, err / np.maximum(floor, 1e-300), 0.0)))
            raise GateFailure(f"query {i}: {int(bad.sum())} scores beyond the fp32 accumulation bound; token {j}: "
                              f"err {err[j]:.3g} > {floor[j]:.3g} (score {o[j]:.6g})")
        bad = err > tol * np.abs(o) + floor
        if bad.any():
            j = int(np.argmax(bad))
            raise GateFailure(f"query {i}: {int(bad.sum())} scores beyond the relative tolerance {tol}; token {j}: "
                              f"err {err[j]:.3g} (score {o[j]:.6g})")
        zero = o == 0.0
        if not np.all(g[zero] == 0.0):
            raise GateFailure(f"query {i}: {int((g[zero] != 0).sum())} exact zero scores are not zero")
        worst_cond = max(worst_cond, float((err / np.maximum(cond, 1e-300)).max()))
        nz = o != 0.0
        if nz.any():
            rel = err[nz] / np.abs(o[nz])
            worst_rel = max(worst_rel, float(rel.max()))
            upper = np.abs(o[nz]) >= np.median(np.abs(o[nz]))
            worst_rel_upper = max(worst_rel_upper, float(rel[upper].max()))
        checked += n
    return {"worst_err_over_cond": worst_cond, "worst_plain_rel": worst_rel,
            "worst_plain_rel_upper_half": worst_rel_upper, "checked": checked, "gamma": gamma}


def check_attention(gpu_o, gpu_lse, ref_o, ref_lse, tol):
    gpu_o = gpu_o.astype(np.float64)
    num = np.linalg.norm(gpu_o - ref_o, axis=-1)
    den = np.linalg.norm(ref_o, axis=-1)
    zero = den == 0
    if not np.all(num[zero] == 0):
        raise GateFailure("output should be exactly 0 where no row is kept")
    rel = num[~zero] / den[~zero]
    worst = float(rel.max()) if rel.size else 0.0
    if worst > tol:
        raise GateFailure(f"attention output relative error {worst:.3g} > {tol}")
    if gpu_lse is not None:
        g = gpu_lse.astype(np.float64)
        inf = np.isneginf(ref_lse)
        if not np.all(np.isneginf(g[inf])):
            raise GateFailure("lse should be -inf where no row is kept")
        d = np.abs(g[~inf] - ref_lse[~inf])
        if not np.all(d <= tol * np.maximum(1.0, np.abs(ref_lse[~inf]))):
            raise GateFailure(f"lse error {d.max():.3g}")
    return worst


def check_selection_near_ties(p, got_idx: np.ndarray, ref_idx: np.ndarray, ref_scores: np.ndarray,
                              rows=None, conds=None) -> dict:
    """End-to-end index gate.  Each row's kept set may differ from the oracle's
    own chain only by tokens whose oracle score lies within the accumulation
    bound (of both tokens) of the row's k-th oracle score: a swap the score
    tolerance allows.  Returns the rows that differ and the largest such gap
    in units of the bound."""
    gamma = accumulation_gamma(p.idx_dim, p.idx_heads)
    rows = range(p.n_q) if rows is None else rows
    differ = 0
    worst = 0.0
    memo = {}
    for r, i in enumerate(rows):
        n = int(p.q_len[i])
        a = set(int(t) for t in got_idx[r] if t >= 0)
        b = set(int(t) for t in ref_idx[r] if t >= 0)
        if len(a) != len(b) or len(a) != min(n, p.topk):
            raise GateFailure(f"query {i}: kept {len(a)} tokens, oracle {len(b)}, expected {min(n, p.topk)}")
        sym = a ^ b
        if not sym:
            continue
        differ += 1
        s = ref_scores[r, :n]
        cond = score_condition(p, i, memo) if conds is None else conds[r]
        kept = ref_idx[r][ref_idx[r] >= 0]
        kth = int(kept[np.argmin(s[kept])])
        for t in sym:
            allowed = gamma * (cond[t] + cond[kth])
            gap = abs(s[t] - s[kth])
            if gap > allowed:
                raise GateFailure(f"query {i}: token {t} kept by one side only, oracle score {s[t]:.9g} is "
                                  f"{gap:.3g} from the k-th score {s[kth]:.9g} (allowed {allowed:.3g})")
            worst = max(worst, gap / allowed if allowed > 0 else 0.0)
    return {"rows_differing": differ, "worst_gap_over_bound": worst}

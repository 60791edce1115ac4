"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (dsa_decode_step with its own workspace for decode; the three entry points
over all 2048 queries for the prefill chunk).

Decode workloads are checked completely against the oracle (every score, every
index, every attention row).  The prefill chunk is too large for the fp64
oracle to score every row in seconds, so sampled rows are checked against the
oracle one by one, and properties that hold at any size are checked on every row.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_14_amd as dsa
from sparse_attention_14_amd import device, inputs

from gpu_util import TOL, check_attention, check_scores, check_selection_near_ties, fmt_scores, gpu_decode_step

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _check_decode(p, dp):
    out, lse, scores, idx, ws = gpu_decode_step(dp)
    g_scores = scores.cpu().numpy()
    ref_scores = oracle.index_scores(p.q_idx, p.q_idx_dtype, p.w_idx, p.keys, p.q_seq, p.q_len)
    worst_s = check_scores(p, g_scores, ref_scores)
    g_idx = idx.cpu().numpy()
    ref_idx, ref_cnt = oracle.topk(g_scores.astype(np.float64), p.q_len, p.topk)
    assert np.array_equal(g_idx, ref_idx)
    ref_o, ref_l, _ = oracle.mla_attend(p.q_mla, p.q_mla_dtype, p.latent, p.kv_lora, g_idx, p.q_seq, p.softmax_scale)
    worst_a = check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, TOL[p.latent.dtype])
    # the oracle's own chain (its scores -> its top-k): the kept sets may differ
    # only by near-ties the score tolerance allows
    own_idx, _ = oracle.topk(ref_scores, p.q_len, p.topk)
    sel = check_selection_near_ties(p, g_idx, own_idx, ref_scores)
    print(f"  {fmt_scores(worst_s)}; worst attention relative error {worst_a:.3g}; rows whose kept set differs from "
          f"the oracle's own chain: {sel['rows_differing']} (worst gap {sel['worst_gap_over_bound']:.3g} x bound)",
          flush=True)
    return g_scores, g_idx


@pytest.mark.parametrize("name", ["glm5_decode_8k", "paged_decode_16x16k_32k", "decode_128k_fp8"])
def test_decode_full_size(name):
    wl = inputs.FULL_WORKLOADS[name]
    print(f"case {name}: full size", flush=True)
    p = inputs.make_problem(wl)
    dp = device.upload(p)
    g_scores, _ = _check_decode(p, dp)
    # injected ties (copied key bytes and scale) must score bit-identically
    for b, (dst, src) in p.meta["ties"].items():
        assert np.array_equal(g_scores[b, dst].view(np.uint32), g_scores[b, src].view(np.uint32)), \
            f"sequence {b}: copied keys do not score identically"


def test_prefill_chunk_full_size_sampled():
    wl = inputs.PREFILL_64K
    print("case prefill_chunk_2048_at_64k: full size, sampled rows", flush=True)
    p = inputs.make_problem(wl)
    dp = device.upload(p)
    n_q, max_len, k = p.n_q, p.max_len, p.topk
    scores = torch.empty(n_q, max_len, device="cuda")
    dsa.dsa_index_scores(scores, dp.q_idx, p.q_idx_dtype, dp.w_idx, dp.keys, dp.q_len, p.idx_heads, max_len,
                         q_seq=dp.q_seq)
    idx = torch.full((n_q, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((n_q,), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(dsa.dsa_topk_workspace_size(n_q, k, max_len), dtype=torch.uint8, device="cuda")
    dsa.dsa_topk(idx, cnt, scores, dp.q_len, k, max_len, workspace=ws)
    out = torch.empty(n_q, p.mla_heads, p.kv_lora, device="cuda")
    lse = torch.empty(n_q, p.mla_heads, device="cuda")
    wa = torch.zeros(max(dsa.mla_sparse_attend_workspace_size(n_q, p.mla_heads, p.kv_lora, k), 1),
                     dtype=torch.uint8, device="cuda")
    dsa.mla_sparse_attend(out, lse, dp.q_mla, p.q_mla_dtype, dp.latent, p.kv_lora, idx, p.softmax_scale,
                          q_seq=dp.q_seq, workspace=wa)
    torch.cuda.synchronize()
    g_scores = scores.cpu().numpy()
    g_idx = idx.cpu().numpy()
    g_cnt = cnt.cpu().numpy()
    lens = p.q_len.astype(np.int64)

    # properties on every row: count = k (every row has n > k), indices strictly
    # ascending inside [0, n), and every kept score >= every dropped score
    assert np.all(g_cnt == k)
    assert np.all(np.diff(g_idx, axis=1) > 0)
    assert np.all(g_idx[:, 0] >= 0) and np.all(g_idx[:, -1] < lens)
    for i in range(n_q):
        row = g_scores[i, :lens[i]]
        kept = np.zeros(lens[i], bool)
        kept[g_idx[i]] = True
        t = row[kept].min()
        assert t >= row[~kept].max(), f"row {i}: a dropped score exceeds a kept one"
        # ties at the boundary go to the lower index
        tied_drop = np.flatnonzero(~kept & (row == t))
        if tied_drop.size:
            assert np.flatnonzero(kept & (row == t)).max() < tied_drop.min(), f"row {i}: tie kept a higher index"
    assert torch.isfinite(out).all().item() and torch.isfinite(lse).all().item()

    # sampled rows against the oracle: scores, indices (all 64 sampled rows), attention
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, n_q - 1], rng.choice(n_q, 62, replace=False)]))
    ref_idx, _ = oracle.topk(g_scores[rows].astype(np.float64), lens[rows].astype(np.int32), k)
    assert np.array_equal(g_idx[rows], ref_idx)
    srows = rows
    ref_s = oracle.index_scores(p.q_idx[srows], p.q_idx_dtype, p.w_idx[srows], p.keys, p.q_seq[srows],
                                p.q_len[srows])
    rs = check_scores(p, g_scores[srows], ref_s, rows=srows)
    print("  " + fmt_scores(rs))
    ref_o, ref_l, _ = oracle.mla_attend(p.q_mla[srows], p.q_mla_dtype, p.latent, p.kv_lora, g_idx[srows],
                                        p.q_seq[srows], p.softmax_scale)
    worst = check_attention(out.cpu().numpy()[srows], lse.cpu().numpy()[srows], ref_o, ref_l, TOL[p.latent.dtype])
    print(f"  sampled rows {len(rows)} (indices), {len(srows)} (scores, attention); attention worst {worst:.3g}")


def test_prefill_chunk_fp8_latent_attention_sampled():
    """The 2048-query chunk's sparse MLA over an fp8 latent cache (the 64-head
    kernel with fp8 rows, 64 steps per query): sampled rows against the oracle."""
    wl = dataclasses.replace(inputs.PREFILL_64K, latent_dtype="e4m3fn")
    print("case prefill_chunk_2048_at_64k, fp8 latent: full size, sampled rows", flush=True)
    p = inputs.make_problem(wl)
    dp = device.upload(p)
    n_q, max_len, k = p.n_q, p.max_len, p.topk
    scores = torch.empty(n_q, max_len, device="cuda")
    dsa.dsa_index_scores(scores, dp.q_idx, p.q_idx_dtype, dp.w_idx, dp.keys, dp.q_len, p.idx_heads, max_len,
                         q_seq=dp.q_seq)
    idx = torch.empty(n_q, k, dtype=torch.int32, device="cuda")
    ws = torch.zeros(dsa.dsa_topk_workspace_size(n_q, k, max_len), dtype=torch.uint8, device="cuda")
    dsa.dsa_topk(idx, None, scores, dp.q_len, k, max_len, workspace=ws)
    del scores
    out = torch.empty(n_q, p.mla_heads, p.kv_lora, device="cuda")
    lse = torch.empty(n_q, p.mla_heads, device="cuda")
    wa = torch.zeros(max(dsa.mla_sparse_attend_workspace_size(n_q, p.mla_heads, p.kv_lora, k), 1),
                     dtype=torch.uint8, device="cuda")
    dsa.mla_sparse_attend(out, lse, dp.q_mla, p.q_mla_dtype, dp.latent, p.kv_lora, idx, p.softmax_scale,
                          q_seq=dp.q_seq, workspace=wa)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item() and torch.isfinite(lse).all().item()
    g_idx = idx.cpu().numpy()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, n_q - 1], rng.choice(n_q, 14, replace=False)]))
    ref_o, ref_l, _ = oracle.mla_attend(p.q_mla[rows], p.q_mla_dtype, p.latent, p.kv_lora, g_idx[rows],
                                        p.q_seq[rows], p.softmax_scale)
    worst = check_attention(out.cpu().numpy()[rows], lse.cpu().numpy()[rows], ref_o, ref_l, TOL[p.latent.dtype])
    print(f"  sampled rows {len(rows)}; attention worst {worst:.3g}")


@pytest.mark.parametrize("name", ["decode_128k_fp8_window4", "paged_decode_16x16k_32k_window4"])
def test_decode_window_full_size(name):
    """The multi-token window workloads in full, as bench.py runs the first:
    every score, index and attention row against the oracle."""
    from gpu_util import gpu_decode_window
    wl = inputs.WINDOW_WORKLOADS[name]
    print(f"case {name}: full size", flush=True)
    p = inputs.make_problem(wl)
    dp = device.upload(p)
    out, lse, scores, idx, ws = gpu_decode_window(dp)
    g_scores = scores.cpu().numpy()
    ref_scores = oracle.index_scores(p.q_idx, p.q_idx_dtype, p.w_idx, p.keys, p.q_seq, p.q_len,
                                     ld=g_scores.shape[1])
    worst_s = check_scores(p, g_scores, ref_scores)
    g_idx = idx.cpu().numpy()
    ref_idx, _ = oracle.topk(g_scores.astype(np.float64), p.q_len, p.topk)
    assert np.array_equal(g_idx, ref_idx)
    ref_o, ref_l, _ = oracle.mla_attend(p.q_mla, p.q_mla_dtype, p.latent, p.kv_lora, g_idx, p.q_seq, p.softmax_scale)
    worst_a = check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, TOL[p.latent.dtype])
    own_idx, _ = oracle.topk(ref_scores, p.q_len, p.topk)
    sel = check_selection_near_ties(p, g_idx, own_idx, ref_scores)
    print(f"  {fmt_scores(worst_s)}; worst attention relative error {worst_a:.3g}; rows whose kept set differs from "
          f"the oracle's own chain: {sel['rows_differing']}", flush=True)


def test_decode_fp8_latent_full_size():
    """The fp8-latent 128K batch in full, as bench.py runs it."""
    wl = inputs.DECODE_128K_FP8_LAT8
    print(f"case {wl.name}: full size", flush=True)
    p = inputs.make_problem(wl)
    dp = device.upload(p)
    _check_decode(p, dp)

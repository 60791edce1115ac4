"""GPU check that a decode step at position p reproduces row p of a prefill
chunk over the same cache (the check pattern of the GLM Reduce model card,
section "Attention implementation": a cached decode step against the full
prefix).

The prefill chunk runs the three entry points over 128 queries (the
GEMM-shaped score kernel, one top-k workgroup per row, the 64-head attention
kernel); the decode step runs sampled rows as sequences of their own over an
aliased view of the same cache (the decode score kernel with its candidate
bounds, the spread top-k, the 16-head attention kernel with a split merge).
Both score kernels compute every score as the same fp32 sum in the same
order, so the scores must agree bit for bit, the kept indices exactly, and
both attention outputs must match the oracle on those indices."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_14_amd as dsa
from sparse_attention_14_amd import device, inputs
from sparse_attention_14_amd.binding import DeviceCache

from gpu_util import TOL, check_attention, check_scores, fmt_scores

pytestmark = pytest.mark.gpu

S = inputs.small
CASES = {
    # rows past 8192 tokens: the decode step spreads each row's top-k over several workgroups
    "bf16_20k": S(inputs.PREFILL_64K, name="dp1", wid=620, seq_len=(20000, 20000), prefill_queries=128),
    "bf16_3k": S(inputs.PREFILL_64K, name="dp2", wid=621, seq_len=(3000, 3000), prefill_queries=96),
}


def _paged_view(cache: DeviceCache, batch: int, n: int) -> DeviceCache:
    """A one-sequence contiguous cache seen as 64-token blocks, every one of
    `batch` sequences mapped onto the same blocks."""
    nb = (n + 63) // 64
    table = torch.arange(nb, dtype=torch.int32, device="cuda").repeat(batch, 1).contiguous()
    rs = cache.desc.row_stride
    return DeviceCache(cache.rows, cache.dtype, cache.width, 64, rs, 64 * rs, scale=cache.scale,
                       scale_block_stride=64, block_table=table)


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_at_position_matches_prefill_row(name):
    p = inputs.make_problem(CASES[name])
    assert not p.decode and np.all(p.q_seq == 0)
    dp = device.upload(p)
    n_q, k, H, L, max_len = p.n_q, p.topk, p.mla_heads, p.kv_lora, p.max_len
    print(f"case {name}: {n_q} queries at positions {int(p.q_len[0]) - 1}..{int(p.q_len[-1]) - 1}", flush=True)

    # prefill chunk
    sc = torch.full((n_q, max_len), float("nan"), device="cuda")
    dsa.dsa_index_scores(sc, dp.q_idx, p.q_idx_dtype, dp.w_idx, dp.keys, dp.q_len, p.idx_heads, max_len,
                         q_seq=dp.q_seq)
    ix = torch.full((n_q, k), -7, dtype=torch.int32, device="cuda")
    tws = torch.zeros(max(dsa.dsa_topk_workspace_size(n_q, k, max_len), 1), dtype=torch.uint8, device="cuda")
    dsa.dsa_topk(ix, None, sc, dp.q_len, k, max_len, workspace=tws)
    out = torch.full((n_q, H, L), float("nan"), device="cuda")
    lse = torch.full((n_q, H), float("nan"), device="cuda")
    aws = torch.zeros(max(dsa.mla_sparse_attend_workspace_size(n_q, H, L, k), 1), dtype=torch.uint8, device="cuda")
    dsa.mla_sparse_attend(out, lse, dp.q_mla, p.q_mla_dtype, dp.latent, L, ix, p.softmax_scale, q_seq=dp.q_seq,
                          workspace=aws)

    # decode steps at sampled positions, one sequence per sampled row
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, n_q - 1], rng.choice(n_q, 6, replace=False)]))
    B = len(rows)
    sel = torch.as_tensor(rows.astype(np.int64), device="cuda")
    keys_b = _paged_view(dp.keys, B, max_len)
    lat_b = _paged_view(dp.latent, B, max_len)
    seq_len = dp.q_len[sel].contiguous()
    d_out = torch.full((B, H, L), float("nan"), device="cuda")
    d_lse = torch.full((B, H), float("nan"), device="cuda")
    d_sc = torch.full((B, max_len), float("nan"), device="cuda")
    d_ix = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(dsa.dsa_decode_step_workspace_size(B, max_len, k, H, L), dtype=torch.uint8, device="cuda")
    dsa.dsa_decode_step(d_out, d_lse, dp.q_idx[sel].contiguous(), p.q_idx_dtype, dp.w_idx[sel].contiguous(), keys_b,
                        dp.q_mla[sel].contiguous(), p.q_mla_dtype, lat_b, L, seq_len, max_len, k, p.softmax_scale, ws,
                        scores_out=d_sc, indices_out=d_ix)
    torch.cuda.synchronize()

    g_sc, g_ix = sc.cpu().numpy(), ix.cpu().numpy()
    h_sc, h_ix = d_sc.cpu().numpy(), d_ix.cpu().numpy()
    for b, r in enumerate(rows):
        n = int(p.q_len[r])
        assert np.array_equal(h_sc[b, :n].view(np.uint32), g_sc[r, :n].view(np.uint32)), \
            f"row {r}: decode scores differ from the prefill row"
        assert np.array_equal(h_ix[b], g_ix[r]), f"row {r}: decode kept indices differ from the prefill row"

    # both against the oracle on the sampled rows
    ref_s = oracle.index_scores(p.q_idx[rows], p.q_idx_dtype, p.w_idx[rows], p.keys, p.q_seq[rows], p.q_len[rows])
    r = check_scores(p, g_sc[rows], ref_s, rows=rows)
    ref_idx, _ = oracle.topk(g_sc[rows].astype(np.float64), p.q_len[rows], k)
    assert np.array_equal(g_ix[rows], ref_idx)
    ref_o, ref_l, _ = oracle.mla_attend(p.q_mla[rows], p.q_mla_dtype, p.latent, L, g_ix[rows], p.q_seq[rows],
                                        p.softmax_scale)
    wp = check_attention(out.cpu().numpy()[rows], lse.cpu().numpy()[rows], ref_o, ref_l, TOL[p.latent.dtype])
    wd = check_attention(d_out.cpu().numpy(), d_lse.cpu().numpy(), ref_o, ref_l, TOL[p.latent.dtype])
    print(f"  {fmt_scores(r)}; attention worst relative error prefill {wp:.3g}, decode {wd:.3g}")


def test_many_positions_decode_equals_prefill():
    """520 positions at once: both sides take their top-k with the many-row
    kernel (the prefill chunk with sampled bounds, the decode step with the
    score kernel's bounds); every row's scores and kept indices must agree bit
    for bit, the prefill top-k must equal the oracle's top-k of its scores on
    every row, scores must match the oracle on sampled rows and attention on a
    few."""
    p = inputs.make_problem(S(inputs.PREFILL_64K, name="dp3", wid=622, seq_len=(9000, 9000), prefill_queries=520))
    dp = device.upload(p)
    n_q, k, H, L, max_len = p.n_q, p.topk, p.mla_heads, p.kv_lora, p.max_len
    print(f"case dp3: {n_q} queries at positions {int(p.q_len[0]) - 1}..{int(p.q_len[-1]) - 1}", flush=True)
    sc = torch.full((n_q, max_len), float("nan"), device="cuda")
    dsa.dsa_index_scores(sc, dp.q_idx, p.q_idx_dtype, dp.w_idx, dp.keys, dp.q_len, p.idx_heads, max_len,
                         q_seq=dp.q_seq)
    ix = torch.full((n_q, k), -7, dtype=torch.int32, device="cuda")
    tws = torch.zeros(max(dsa.dsa_topk_workspace_size(n_q, k, max_len), 1), dtype=torch.uint8, device="cuda")
    dsa.dsa_topk(ix, None, sc, dp.q_len, k, max_len, workspace=tws)

    keys_b = _paged_view(dp.keys, n_q, max_len)
    lat_b = _paged_view(dp.latent, n_q, max_len)
    d_out = torch.full((n_q, H, L), float("nan"), device="cuda")
    d_lse = torch.full((n_q, H), float("nan"), device="cuda")
    d_sc = torch.full((n_q, max_len), float("nan"), device="cuda")
    d_ix = torch.full((n_q, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(dsa.dsa_decode_step_workspace_size(n_q, max_len, k, H, L), dtype=torch.uint8, device="cuda")
    dsa.dsa_decode_step(d_out, d_lse, dp.q_idx, p.q_idx_dtype, dp.w_idx, keys_b, dp.q_mla, p.q_mla_dtype, lat_b, L,
                        dp.q_len, max_len, k, p.softmax_scale, ws, scores_out=d_sc, indices_out=d_ix)
    torch.cuda.synchronize()

    g_sc, g_ix = sc.cpu().numpy(), ix.cpu().numpy()
    h_sc, h_ix = d_sc.cpu().numpy(), d_ix.cpu().numpy()
    for r in range(n_q):
        n = int(p.q_len[r])
        assert np.array_equal(h_sc[r, :n].view(np.uint32), g_sc[r, :n].view(np.uint32)), \
            f"row {r}: decode scores differ from the prefill row"
    assert np.array_equal(h_ix, g_ix), "decode kept indices differ from the prefill rows"
    ref_idx, _ = oracle.topk(g_sc.astype(np.float64), p.q_len, k)
    assert np.array_equal(g_ix, ref_idx)
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, n_q - 1], rng.choice(n_q, 10, replace=False)]))
    ref_s = oracle.index_scores(p.q_idx[rows], p.q_idx_dtype, p.w_idx[rows], p.keys, p.q_seq[rows], p.q_len[rows])
    r = check_scores(p, g_sc[rows], ref_s, rows=rows)
    few = rows[:4]
    ref_o, ref_l, _ = oracle.mla_attend(p.q_mla[few], p.q_mla_dtype, p.latent, L, g_ix[few], p.q_seq[few],
                                        p.softmax_scale)
    wd = check_attention(d_out.cpu().numpy()[few], d_lse.cpu().numpy()[few], ref_o, ref_l, TOL[p.latent.dtype])
    print(f"  {fmt_scores(r)}; decode attention worst relative error {wd:.3g}")

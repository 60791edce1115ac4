"""GPU parity of the multi-token decode window (dsa_decode_window): the known
token and the guesses after it go through the path together, query j of a
sequence of n tokens at position n - window + j.

- stage by stage against the oracle (scores within tolerance, indices
  bit-exact against the oracle's top-k of the GPU's scores, attention within
  tolerance), including windows longer than a sequence (queries that see
  nothing);
- bit-identical to single-token steps: on a paged cache, a second block table
  that gives every window query a sequence of its own (aliasing its
  sequence's blocks) turns the window into an ordinary dsa_decode_step of
  batch * window queries, each ending at its own position; every output must
  match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_14_amd as dsa
from sparse_attention_14_amd import device, inputs
from sparse_attention_14_amd.binding import DeviceCache

from gpu_util import TOL, check_attention, check_scores, gpu_decode_window

pytestmark = pytest.mark.gpu

S = inputs.small
CASES = {
    "fp8_w4": S(inputs.DECODE_128K_FP8_W4, name="w1", wid=501, batch=2, seq_len=(10000, 10000)),
    "bf16_paged_w3": S(inputs.PAGED_DECODE_W4, name="w2", wid=502, batch=3, seq_len=(100, 9000), window=3),
    "fp8_w4_bounded": S(inputs.DECODE_128K_FP8_W4, name="w3", wid=503, batch=2, seq_len=(30000, 40000)),
    "bf16_w8_short": S(inputs.DECODE_8K, name="w4", wid=504, batch=3, seq_len=(2, 2100), window=8),
    "bf16_w8_tiny": S(inputs.DECODE_8K, name="w6", wid=506, batch=2, seq_len=(3, 3), window=8),
    "bf16_paged_w4_bounded": S(inputs.PAGED_DECODE_W4, name="w5", wid=505, batch=2, seq_len=(13000, 26000)),
    "fp8_latent8_w4": S(inputs.DECODE_128K_FP8_LAT8, name="w7", wid=507, batch=4, seq_len=(3000, 9000), window=4),
    # windows of 2 and 6: query pairs that do not share a workgroup with another pair
    "fp8_w6": S(inputs.DECODE_128K_FP8_W4, name="w9", wid=509, batch=2, seq_len=(5000, 12000), window=6),
    "bf16_paged_w2": S(inputs.PAGED_DECODE_W4, name="w10", wid=510, batch=3, seq_len=(700, 20000), window=2),
    # fewer indexer heads than the MFMA's 32 rows (zero q rows and weights in the pair kernel)
    "fp8_w4_h20": S(inputs.DECODE_128K_FP8_W4, name="w11", wid=511, batch=2, seq_len=(3000, 7000), idx_heads=20),
    # fp32 indexer queries: the window rows come from their own kernel
    "f32_w3": S(inputs.TINY_FP32, name="w8", wid=508, batch=3, seq_len=(2, 900), window=3),
}


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    p = inputs.make_problem(CASES[request.param])
    return p, device.upload(p)


def test_decode_window_stages(case):
    p, dp = case
    W = p.meta["workload"].window
    print(f"case {p.name}: window={W} lens={list(p.meta['seq_lens'])} q_len={p.q_len.tolist()}", flush=True)
    out, lse, scores, idx, ws = gpu_decode_window(dp)
    g_scores = scores.cpu().numpy()
    ref_scores = oracle.index_scores(p.q_idx, p.q_idx_dtype, p.w_idx, p.keys, p.q_seq, p.q_len)
    check_scores(p, g_scores, ref_scores)
    g_idx = idx.cpu().numpy()
    ref_idx, _ = oracle.topk(g_scores.astype(np.float64), p.q_len, p.topk)
    assert np.array_equal(g_idx, ref_idx)
    ref_o, ref_l, _ = oracle.mla_attend(p.q_mla, p.q_mla_dtype, p.latent, p.kv_lora, g_idx, p.q_seq, p.softmax_scale)
    worst = check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, TOL[p.latent.dtype])
    # queries before the sequence start see nothing
    empty = p.q_len == 0
    if empty.any():
        assert np.all(g_idx[empty] == -1)
        assert np.all(out.cpu().numpy()[empty] == 0.0) and np.all(np.isneginf(lse.cpu().numpy()[empty]))
    print(f"  attention worst relative error {worst:.3g}; empty queries {int(empty.sum())}")


def _aliased(cache: DeviceCache, row_seq: np.ndarray) -> DeviceCache:
    """The same storage with one block-table row per window query (its sequence's row)."""
    table = cache.block_table[torch.as_tensor(row_seq.astype(np.int64), device="cuda")].contiguous()
    return DeviceCache(cache.rows, cache.dtype, cache.width, cache.block_size, cache.desc.row_stride,
                       cache.desc.block_stride, scale=cache.scale, scale_block_stride=cache.desc.scale_block_stride,
                       block_table=table)


@pytest.mark.parametrize("name", ["bf16_paged_w3", "bf16_paged_w4_bounded", "bf16_paged_w2"])
def test_decode_window_equals_single_token_steps(name):
    p = inputs.make_problem(CASES[name])
    dp = device.upload(p)
    out, lse, scores, idx, _ = gpu_decode_window(dp)
    keys1, lat1 = _aliased(dp.keys, p.q_seq), _aliased(dp.latent, p.q_seq)
    n_q, H, L = p.n_q, p.mla_heads, p.kv_lora
    max_len = scores.shape[1]
    o1 = torch.full_like(out, float("nan"))
    l1 = torch.full_like(lse, float("nan"))
    s1 = torch.full_like(scores, float("nan"))
    i1 = torch.full_like(idx, -7)
    ws = torch.zeros(dsa.dsa_decode_step_workspace_size(n_q, max_len, p.topk, H, L), dtype=torch.uint8, device="cuda")
    dsa.dsa_decode_step(o1, l1, dp.q_idx, p.q_idx_dtype, dp.w_idx, keys1, dp.q_mla, p.q_mla_dtype, lat1, L, dp.q_len,
                        max_len, p.topk, p.softmax_scale, ws, scores_out=s1, indices_out=i1)
    torch.cuda.synchronize()
    for i in range(n_q):
        n = int(p.q_len[i])
        assert torch.equal(scores[i, :n].view(torch.int32), s1[i, :n].view(torch.int32)), f"scores of query {i}"
    assert torch.equal(idx, i1)
    assert torch.equal(out.view(torch.int32), o1.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), l1.view(torch.int32))

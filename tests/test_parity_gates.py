"""The parity gates (parity_gates.py) against plausible kernel mistakes, on the
CPU.  Each mistake is planted in the oracle's computation (or its output), and
the gate must reject it; an honest fp32-accumulated computation of the same
scores must pass.  This shows the score gate is tight enough to catch, among
others, scores stored rounded to bf16 and a head that loses one of its 128
dimensions, which a condition-scaled bound of 2e-3 would let through."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_14_amd import inputs

from parity_gates import (GateFailure, accumulation_gamma, check_scores, check_selection_near_ties, decode_values,
                          logical_rows)

S = inputs.small
WORKLOADS = {
    "fp8_keys": S(inputs.DECODE_128K_FP8, name="g1", wid=601, batch=2, seq_len=(3000, 4000)),
    "bf16_keys": S(inputs.DECODE_8K, name="g2", wid=602, batch=2, seq_len=(2500, 3500)),
    "f32_keys": inputs.TINY_FP32,
    "bf16_signed_w": S(inputs.DECODE_8K, name="g3", wid=603, batch=2, seq_len=(1500, 2000), idx_heads=7, w_lo=-1.0,
                       w_hi=1.0),
}


@pytest.fixture(scope="module", params=sorted(WORKLOADS))
def case(request):
    p = inputs.make_problem(WORKLOADS[request.param])
    ref = oracle.index_scores(p.q_idx, p.q_idx_dtype, p.w_idx, p.keys, p.q_seq, p.q_len)
    return p, ref


def fp32_scores(p, relu_after_sum=False):
    """The scores computed the way a kernel would: float32 products and sums
    (torch CPU float32 matmul), ReLU per head, float32 weighted head sum."""
    out = np.full((p.n_q, p.max_len), np.nan, dtype=np.float32)
    for i in range(p.n_q):
        n = int(p.q_len[i])
        k = torch.from_numpy(logical_rows(p.keys, int(p.q_seq[i]), n).astype(np.float32))
        q = torch.from_numpy(decode_values(p.q_idx[i].reshape(-1), p.q_idx_dtype)
                             .reshape(p.idx_heads, p.idx_dim).astype(np.float32))
        w = torch.from_numpy(p.w_idx[i].astype(np.float32))
        dots = q @ k.T                                       # [H, n] float32
        if relu_after_sum:
            s = torch.clamp(w @ dots, min=0.0)
        else:
            s = w @ torch.clamp(dots, min=0.0)
        out[i, :n] = s.numpy()
    return out


def test_fp32_accumulated_scores_pass(case):
    p, ref = case
    r = check_scores(p, fp32_scores(p), ref)
    assert r["worst_err_over_cond"] <= accumulation_gamma(p.idx_dim, p.idx_heads)
    # the oracle's own values rounded once to float32 pass with a wide margin
    r = check_scores(p, ref.astype(np.float32), ref)
    assert r["worst_err_over_cond"] <= 2.0 ** -24


def test_bf16_rounded_scores_fail(case):
    p, ref = case
    g = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).float().numpy()
    with pytest.raises(GateFailure):
        check_scores(p, g, ref)


def test_dropped_dimension_fails(case):
    """One head loses one dimension of its dot product."""
    p, ref = case
    q = p.q_idx.copy()
    q.reshape(p.n_q, p.idx_heads, p.idx_dim)[:, p.idx_heads // 2, p.idx_dim - 3] = 0
    bad = oracle.index_scores(q, p.q_idx_dtype, p.w_idx, p.keys, p.q_seq, p.q_len)
    with pytest.raises(GateFailure):
        check_scores(p, bad, ref)


def test_swapped_head_weights_fail(case):
    p, ref = case
    w = p.w_idx.copy()
    w[:, [0, 1]] = w[:, [1, 0]]
    bad = oracle.index_scores(p.q_idx, p.q_idx_dtype, w, p.keys, p.q_seq, p.q_len)
    with pytest.raises(GateFailure):
        check_scores(p, bad, ref)


def test_relu_after_the_head_sum_fails(case):
    p, ref = case
    with pytest.raises(GateFailure):
        check_scores(p, fp32_scores(p, relu_after_sum=True), ref)


def test_scale_not_applied_fails():
    p = inputs.make_problem(WORKLOADS["fp8_keys"])
    ref = oracle.index_scores(p.q_idx, p.q_idx_dtype, p.w_idx, p.keys, p.q_seq, p.q_len)
    import copy
    keys = copy.copy(p.keys)
    keys.scale = np.ones_like(p.keys.scale)
    bad = oracle.index_scores(p.q_idx, p.q_idx_dtype, p.w_idx, keys, p.q_seq, p.q_len)
    with pytest.raises(GateFailure):
        check_scores(p, bad, ref)


def test_shifted_token_fails(case):
    p, ref = case
    bad = ref.copy()
    n = int(p.q_len[0])
    bad[0, 1:n] = ref[0, 0:n - 1]
    with pytest.raises(GateFailure):
        check_scores(p, bad, ref)


def test_nonzero_where_every_head_is_negative_fails():
    p = inputs.make_problem(WORKLOADS["bf16_signed_w"])   # 7 heads: some tokens have every dot product <= 0
    ref = oracle.index_scores(p.q_idx, p.q_idx_dtype, p.w_idx, p.keys, p.q_seq, p.q_len)
    zeros = np.flatnonzero(ref[0, :p.q_len[0]] == 0.0)
    if zeros.size == 0:
        pytest.skip("no exact-zero score in this draw")
    bad = ref.copy()
    bad[0, zeros[0]] = 1e-30
    with pytest.raises(GateFailure):
        check_scores(p, bad, ref)


def test_selection_gate():
    """Kept sets that differ by a near-tie pass; a swap far from the boundary fails."""
    p = inputs.make_problem(WORKLOADS["bf16_keys"])
    ref = oracle.index_scores(p.q_idx, p.q_idx_dtype, p.w_idx, p.keys, p.q_seq, p.q_len)
    idx, _ = oracle.topk(ref, p.q_len, p.topk)
    assert check_selection_near_ties(p, idx, idx, ref)["rows_differing"] == 0
    # the k-th and (k+1)-th tokens exchanged, with scores made equal up to the bound
    n = int(p.q_len[0])
    order = np.argsort(-ref[0, :n], kind="stable")
    kth, nxt = int(order[p.topk - 1]), int(order[p.topk])
    near = ref.copy()
    near[0, nxt] = near[0, kth]
    swapped = idx.copy()
    row = set(idx[0].tolist()) - {kth} | {nxt}
    swapped[0] = np.sort(np.array(sorted(row), dtype=np.int32))
    assert check_selection_near_ties(p, swapped, idx, near)["rows_differing"] == 1
    # the same exchange with the true scores far apart, or with a low-ranked token, fails
    far = int(order[n - 1])
    row = set(idx[0].tolist()) - {kth} | {far}
    bad = idx.copy()
    bad[0] = np.sort(np.array(sorted(row), dtype=np.int32))
    with pytest.raises(GateFailure):
        check_selection_near_ties(p, bad, idx, ref)

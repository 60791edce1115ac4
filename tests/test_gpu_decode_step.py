"""GPU parity: the fused dsa_decode_step against the oracle, stage by stage
(scores within tolerance; indices bit-exact against the oracle's top-k of the
GPU's scores; attention within tolerance on the GPU's indices), plus the
oracle's own end-to-end chain, determinism and workspace reuse."""
import numpy as np
import pytest
import torch

import sparse_attention_14_amd as dsa

import oracle
from sparse_attention_14_amd import device, inputs

from gpu_util import TOL, check_attention, check_scores, check_selection_near_ties, fmt_scores, gpu_decode_step

pytestmark = pytest.mark.gpu

S = inputs.small
CASES = {
    "tiny_fp32_full": inputs.TINY_FP32,
    "bf16_small": S(inputs.DECODE_8K, name="d1", wid=401, batch=2, seq_len=(1500, 6000)),
    "bf16_paged": S(inputs.PAGED_DECODE, name="d2", wid=402, batch=4, seq_len=(100, 9000)),
    "fp8_ties": S(inputs.DECODE_128K_FP8, name="d3", wid=403, batch=2, seq_len=(10000, 10000)),
    "fp8_short": S(inputs.DECODE_128K_FP8, name="d4", wid=404, batch=3, seq_len=(1, 2100)),
    # long enough (n > the 12288-candidate buffer) for the score kernel's bounds to filter
    "fp8_long_bounded": S(inputs.DECODE_128K_FP8, name="d5", wid=405, batch=2, seq_len=(30000, 40000)),
    "bf16_paged_long_bounded": S(inputs.PAGED_DECODE, name="d6", wid=406, batch=3, seq_len=(13000, 26000)),
    "fp8_latent8": S(inputs.DECODE_128K_FP8_LAT8, name="d8", wid=408, batch=2, seq_len=(5000, 20000)),
}


CASES_BY_NAME = {wl.name: wl for wl in CASES.values()}


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    p = inputs.make_problem(CASES[request.param])
    return p, device.upload(p)


def test_decode_step_stages(case):
    p, dp = case
    print(f"case {p.name}: batch={p.n_q} lens={p.q_len.tolist()} keys={p.keys.dtype}", flush=True)
    out, lse, scores, idx, ws = gpu_decode_step(dp)
    g_scores = scores.cpu().numpy()
    ref_scores = oracle.index_scores(p.q_idx, p.q_idx_dtype, p.w_idx, p.keys, p.q_seq, p.q_len)
    r = check_scores(p, g_scores, ref_scores)
    g_idx = idx.cpu().numpy()
    ref_idx, _ = oracle.topk(g_scores.astype(np.float64), p.q_len, p.topk)
    assert np.array_equal(g_idx, ref_idx)
    ref_o, ref_l, _ = oracle.mla_attend(p.q_mla, p.q_mla_dtype, p.latent, p.kv_lora, g_idx, p.q_seq, p.softmax_scale)
    worst = check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, TOL[p.latent.dtype])
    print(f"  {fmt_scores(r)}; attention worst relative error {worst:.3g}")


def test_decode_step_end_to_end_oracle(case):
    """The oracle's own chain (its scores -> its top-k -> its attention).  A
    row's kept set may differ from the oracle's only by tokens whose oracle
    score is within the fp32 accumulation bound of the row's k-th oracle score
    (a swap the score tolerance allows); rows whose sets agree must match the
    oracle's attention within tolerance."""
    p, dp = case
    out, lse, scores, idx, ws = gpu_decode_step(dp)
    ref = oracle.decode_step(p)
    g_idx = idx.cpu().numpy()
    sel = check_selection_near_ties(p, g_idx, ref["indices"], ref["scores"])
    same = np.array([set(g_idx[i][g_idx[i] >= 0]) == set(ref["indices"][i][ref["indices"][i] >= 0])
                     for i in range(p.n_q)])
    print(f"  rows whose kept set differs from the oracle's own chain: {sel['rows_differing']} / {p.n_q} "
          f"(worst gap {sel['worst_gap_over_bound']:.3g} x bound)")
    assert same.sum() == p.n_q - sel["rows_differing"]
    if CASES_BY_NAME[p.name].tie_fraction == 0:
        # no injected ties: near-ties within the bound are not expected at these sizes
        assert sel["rows_differing"] == 0, "kept sets differ from the oracle's own chain without injected ties"
    if same.any():
        check_attention(out.cpu().numpy()[same], lse.cpu().numpy()[same], ref["out"][same], ref["lse"][same],
                        TOL[p.latent.dtype])


def test_decode_step_is_deterministic_and_workspace_reusable(case):
    p, dp = case
    a = gpu_decode_step(dp)
    b = gpu_decode_step(dp, ws=a[4])           # same workspace again
    for x, y in zip(a[:4], b[:4]):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_key_ties_straddle_the_boundary():
    """Copies of the rank-k token's key bytes and scale (rank by the oracle's
    scores) are planted at 4 earlier and 4 later positions, so the GPU scores
    them bit-identically and the boundary falls inside the tie group."""
    wl = S(inputs.DECODE_128K_FP8, name="d7", wid=407, batch=2, seq_len=(20000, 30000), tie_fraction=0.0)
    p = inputs.make_problem(wl)
    ref = oracle.index_scores(p.q_idx, p.q_idx_dtype, p.w_idx, p.keys, p.q_seq, p.q_len)
    rng = np.random.default_rng(9)
    planted = {}
    for b in range(p.n_q):
        n = int(p.q_len[b])
        order = np.argsort(-ref[b, :n], kind="stable")
        t = int(order[p.topk - 1])
        others = order[p.topk + 50:]       # overwrite only low-ranked tokens
        dst = np.concatenate([rng.choice(others[others < t], 4, replace=False),
                              rng.choice(others[others > t], 4, replace=False)])
        for d in dst:
            inputs.copy_token(p.keys, b, int(d), t)
        planted[b] = (t, dst)
    dp = device.upload(p)
    print(f"case d7: planted boundary ties at {[(b, t) for b, (t, _) in planted.items()]}", flush=True)
    out, lse, scores, idx, ws = gpu_decode_step(dp)
    g_scores = scores.cpu().numpy()
    for b, (t, dst) in planted.items():
        assert np.all(g_scores[b, dst].view(np.uint32) == g_scores[b, t].view(np.uint32))
        v = g_scores[b, t]
        assert (g_scores[b, :p.q_len[b]] > v).sum() < p.topk < (g_scores[b, :p.q_len[b]] >= v).sum()
    ref_idx, _ = oracle.topk(g_scores.astype(np.float64), p.q_len, p.topk)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)


def test_decode_step_graph_replays_match_eager():
    """The step captured in a HIP graph, replayed several times with other eager
    work and synchronisations between replays, gives the eager result bit for bit."""
    p = inputs.make_problem(CASES["fp8_long_bounded"])
    dp = device.upload(p)
    other = device.upload(inputs.make_problem(CASES["fp8_ties"]))
    B, H, L = p.n_q, p.mla_heads, p.kv_lora
    ref = gpu_decode_step(dp)
    out = torch.empty(B, H, L, device="cuda")
    lse = torch.empty(B, H, device="cuda")
    idx = torch.empty(B, p.topk, dtype=torch.int32, device="cuda")
    ws = torch.zeros(dsa.dsa_decode_step_workspace_size(B, p.max_len, p.topk, H, L), dtype=torch.uint8,
                     device="cuda")
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dsa.dsa_decode_step(out, lse, dp.q_idx, p.q_idx_dtype, dp.w_idx, dp.keys, dp.q_mla, p.q_mla_dtype,
                            dp.latent, L, dp.q_len, p.max_len, p.topk, p.softmax_scale, ws, indices_out=idx)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        idx.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[3]), f"replay {rep}: indices differ"
        assert torch.equal(out.view(torch.int32), ref[0].view(torch.int32)), f"replay {rep}: out differs"
        assert torch.equal(lse.view(torch.int32), ref[1].view(torch.int32)), f"replay {rep}: lse differs"
        gpu_decode_step(other)      # unrelated eager work between replays


@pytest.mark.parametrize("wl", [S(inputs.DECODE_128K_FP8, name="d9", wid=409, batch=4, seq_len=(3000, 8000)),
                                S(inputs.PAGED_DECODE, name="d10", wid=410, batch=5, seq_len=(9000, 20000))],
                         ids=["fp8_one_workgroup_rows", "bf16_paged_spread_rows"])
def test_empty_sequences_in_the_batch(wl):
    """Sequences with no tokens (padding slots of a batch): no score written, no
    kept index (-1 padding), output 0 and lse -inf; the other sequences are
    unaffected."""
    p = inputs.make_problem(wl)
    p.q_len[[1, 3]] = 0
    print(f"case {p.name}: lens {p.q_len.tolist()}", flush=True)
    dp = device.upload(p)
    out, lse, scores, idx, ws = gpu_decode_step(dp)
    g_scores = scores.cpu().numpy()
    ref_scores = oracle.index_scores(p.q_idx, p.q_idx_dtype, p.w_idx, p.keys, p.q_seq, p.q_len)
    check_scores(p, g_scores, ref_scores)
    g_idx = idx.cpu().numpy()
    ref_idx, _ = oracle.topk(g_scores.astype(np.float64), p.q_len, p.topk)
    assert np.array_equal(g_idx, ref_idx)
    assert np.all(g_idx[[1, 3]] == -1)
    ref_o, ref_l, _ = oracle.mla_attend(p.q_mla, p.q_mla_dtype, p.latent, p.kv_lora, g_idx, p.q_seq, p.softmax_scale)
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, TOL[p.latent.dtype])
    assert torch.all(out[[1, 3]] == 0).item() and torch.all(torch.isneginf(lse[[1, 3]])).item()

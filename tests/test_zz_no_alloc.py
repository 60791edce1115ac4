"""GPU check of dsa_decode_step_noalloc (the allocation-free decode step on the
library's static per-GPU scratch) against dsa_decode_step with a caller
workspace: two calls in a row, the second with a smaller input, each bit for
bit equal to the workspace version (scores, kept indices, output, lse)."""
import numpy as np
import pytest
import torch

import sparse_attention_14_amd as dsa
from sparse_attention_14_amd import device, inputs

pytestmark = pytest.mark.gpu

S = inputs.small


def _outputs(p):
    B, H, L = p.n_q, p.mla_heads, p.kv_lora
    return (torch.full((B, H, L), float("nan"), device="cuda"), torch.full((B, H), float("nan"), device="cuda"),
            torch.full((B, max(p.max_len, 1)), float("nan"), device="cuda"),
            torch.full((B, p.topk), -7, dtype=torch.int32, device="cuda"))


def _both(p, dp):
    B, H, L = p.n_q, p.mla_heads, p.kv_lora
    ref = _outputs(p)
    ws = torch.zeros(dsa.dsa_decode_step_workspace_size(B, p.max_len, p.topk, H, L), dtype=torch.uint8,
                     device="cuda")
    dsa.dsa_decode_step(ref[0], ref[1], dp.q_idx, p.q_idx_dtype, dp.w_idx, dp.keys, dp.q_mla, p.q_mla_dtype,
                        dp.latent, L, dp.q_len, p.max_len, p.topk, p.softmax_scale, ws, scores_out=ref[2],
                        indices_out=ref[3])
    got = _outputs(p)
    torch.cuda.synchronize()
    dsa.dsa_decode_step_noalloc(got[0], got[1], dp.q_idx, p.q_idx_dtype, dp.w_idx, dp.keys, dp.q_mla, p.q_mla_dtype,
                                dp.latent, L, dp.q_len, p.max_len, p.topk, p.softmax_scale, scores_out=got[2],
                                indices_out=got[3])
    torch.cuda.synchronize()
    return ref, got


def _assert_same(p, ref, got):
    for i in range(p.n_q):
        n = int(p.q_len[i])
        assert torch.equal(ref[2][i, :n].view(torch.int32), got[2][i, :n].view(torch.int32)), f"scores of row {i}"
    assert torch.equal(ref[3], got[3]), "kept indices"
    assert torch.equal(ref[0].view(torch.int32), got[0].view(torch.int32)), "output"
    assert torch.equal(ref[1].view(torch.int32), got[1].view(torch.int32)), "lse"


def test_noalloc_matches_workspace_step_twice_second_smaller():
    big = inputs.make_problem(inputs.DECODE_128K_FP8)            # 4 x 131072, fp8 keys, the bench workload
    small = inputs.make_problem(S(inputs.PAGED_DECODE, name="na2", wid=902, batch=2, seq_len=(3000, 9000)))
    for p in (big, small):
        print(f"case {p.name}: batch {p.n_q} lens {p.q_len.tolist()}", flush=True)
        dp = device.upload(p)
        ref, got = _both(p, dp)
        _assert_same(p, ref, got)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """96 sequences of up to 16384 tokens need about 55 MiB of scratch: the call
    is rejected on the host (DSA_ERR_WORKSPACE_TOO_SMALL) and launches nothing."""
    p = inputs.make_problem(S(inputs.PAGED_DECODE, name="na3", wid=903, batch=2, seq_len=(100, 200)))
    dp = device.upload(p)
    B, H, L = 96, p.mla_heads, p.kv_lora
    assert dsa.dsa_decode_step_workspace_size(B, 16384, p.topk, H, L) > dsa.binding.NOALLOC_SCRATCH_BYTES
    out = torch.empty(B, H, L, device="cuda")
    seq_len = torch.full((B,), 100, dtype=torch.int32, device="cuda")
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_decode_step_noalloc(out, None, dp.q_idx, p.q_idx_dtype, dp.w_idx, dp.keys, dp.q_mla, p.q_mla_dtype,
                                    dp.latent, L, seq_len, 16384, p.topk, p.softmax_scale)
    assert e.value.code == 3

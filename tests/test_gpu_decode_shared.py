"""GPU parity of dsa_decode_shared: a layer that reuses the kept indices an
earlier full layer chose for the same queries ("Self-contained GLM-5 serving
stack", component list: full/shared DSA indexer selection) runs only sparse
attention over its own latent cache.

- against the oracle's attention of the sharing layer over the full layer's
  indices (within tolerance), for single-token steps and windows, including
  queries that keep fewer than k tokens or none;
- a sharing layer given the full layer's own queries and cache reproduces the
  full step's output bit for bit (the same attention kernels and split plan).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_14_amd as dsa
from sparse_attention_14_amd import device, inputs

from gpu_util import TOL, check_attention, gpu_decode_step, gpu_decode_window

pytestmark = pytest.mark.gpu

S = inputs.small
CASES = {
    "fp8_w1": S(inputs.DECODE_128K_FP8, name="s1", wid=601, batch=3, seq_len=(1500, 30000)),
    "bf16_paged_w1": S(inputs.PAGED_DECODE, name="s2", wid=602, batch=4, seq_len=(1, 9000)),
    "fp8_w4": S(inputs.DECODE_128K_FP8_W4, name="s3", wid=603, batch=2, seq_len=(3000, 12000)),
    "bf16_paged_w3_short": S(inputs.PAGED_DECODE_W4, name="s4", wid=604, batch=3, seq_len=(2, 2500), window=3),
    "f32_tiny": inputs.TINY_FP32,
    "fp8_latent8_w1": S(inputs.DECODE_128K_FP8_LAT8, name="s5", wid=605, batch=3, seq_len=(2000, 9000)),
}


def _layers(name):
    """(full layer, sharing layer): the same sequences and keys; the sharing
    layer's latent rows and MLA queries are drawn at other scales, so its
    attention differs from the full layer's."""
    wl = CASES[name]
    full = inputs.make_problem(wl)
    other = inputs.make_problem(dataclasses.replace(wl, latent_sigma=wl.latent_sigma * 1.7,
                                                    q_mla_sigma=wl.q_mla_sigma * 0.6))
    assert np.array_equal(full.q_len, other.q_len)
    return full, other


def _full_step(dp):
    W = dp.host.meta["workload"].window
    return gpu_decode_window(dp) if W > 1 else gpu_decode_step(dp)


def _shared_step(dp, idx):
    p = dp.host
    W = p.meta["workload"].window
    B = len(p.meta["seq_lens"])
    out = torch.full((p.n_q, p.mla_heads, p.kv_lora), float("nan"), device="cuda")
    lse = torch.full((p.n_q, p.mla_heads), float("nan"), device="cuda")
    wsz = dsa.dsa_decode_shared_workspace_size(B, W, idx.shape[1], p.mla_heads, p.kv_lora)
    ws = torch.zeros(max(wsz, 1), dtype=torch.uint8, device="cuda")
    dsa.dsa_decode_shared(out, lse, dp.q_mla, p.q_mla_dtype, dp.latent, p.kv_lora, idx, B, W, p.softmax_scale,
                          workspace=ws)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("name", sorted(CASES))
def test_shared_layer_matches_the_oracle(name):
    full, other = _layers(name)
    print(f"case {name}: {full.n_q} queries, lens {full.q_len.tolist()[:8]}", flush=True)
    dfull = device.upload(full)
    idx = _full_step(dfull)[3]
    dother = device.upload(other)
    out, lse = _shared_step(dother, idx)
    g_idx = idx.cpu().numpy()
    ref_o, ref_l, _ = oracle.mla_attend(other.q_mla, other.q_mla_dtype, other.latent, other.kv_lora, g_idx,
                                        other.q_seq, other.softmax_scale)
    worst = check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, TOL[other.latent.dtype])
    print(f"  worst relative error {worst:.3g}")


@pytest.mark.parametrize("name", ["fp8_w1", "fp8_w4", "bf16_paged_w3_short", "f32_tiny"])
def test_shared_layer_with_the_full_layers_inputs_is_bit_identical(name):
    full, _ = _layers(name)
    dfull = device.upload(full)
    out_f, lse_f, _, idx, _ = _full_step(dfull)
    out_s, lse_s = _shared_step(dfull, idx)
    assert torch.equal(out_s.view(torch.int32), out_f.view(torch.int32))
    assert torch.equal(lse_s.view(torch.int32), lse_f.view(torch.int32))

"""Entry points captured in a HIP graph: a decode layer as a caller would
capture it (cache append -> multi-token window step -> output projection,
then a layer sharing the selection), replayed several times with unrelated
eager work and synchronisations between replays; every replay must give the
eager results bit for bit.  The library records no memset and allocates
nothing, so the captured sequence is exactly the eager one."""
import numpy as np
import pytest
import torch

import sparse_attention_14_amd as dsa
from sparse_attention_14_amd import device, inputs

from gpu_util import gpu_decode_step

pytestmark = pytest.mark.gpu


def _dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def test_captured_window_layer_replays_match_eager():
    wl = inputs.small(inputs.DECODE_128K_FP8_W4, name="g1", wid=801, batch=3, seq_len=(2000, 20000))
    p = inputs.make_problem(wl)
    dp = device.upload(p)
    other = device.upload(inputs.make_problem(inputs.small(inputs.DECODE_8K, name="g2", wid=802, batch=2,
                                                           seq_len=(1000, 3000))))
    W = wl.window
    nk, nl, aseq, apos = inputs.append_tokens(p, W, "bf16")
    t_nk, t_nl, t_seq, t_pos = _dev(nk), _dev(nl), _dev(aseq), _dev(apos)
    aw = inputs.AbsorbWorkload(name="g3", wid=803, n_q=p.n_q)
    x = inputs.make_absorb(aw)
    w_uv = _dev(x["w_uv"])
    seq_len = torch.tensor(np.asarray(p.meta["seq_lens"], dtype=np.int32), device="cuda")
    B, H, L, k = int(seq_len.shape[0]), p.mla_heads, p.kv_lora, p.topk
    max_len = int(max(p.meta["seq_lens"]))
    out = torch.empty(p.n_q, H, L, device="cuda")
    lse = torch.empty(p.n_q, H, device="cuda")
    idx = torch.empty(p.n_q, k, dtype=torch.int32, device="cuda")
    proj = torch.empty(p.n_q, H, aw.d_v, device="cuda")
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    ws = torch.zeros(dsa.dsa_decode_window_workspace_size(B, W, max_len, k, H, L), dtype=torch.uint8, device="cuda")
    ws2 = torch.zeros(max(dsa.dsa_decode_shared_workspace_size(B, W, k, H, L), 1), dtype=torch.uint8, device="cuda")

    def layer():
        dsa.dsa_cache_append(dp.keys, t_nk, "bf16", dp.latent, t_nl, t_pos, seq=t_seq)
        dsa.dsa_decode_window(out, lse, dp.q_idx, p.q_idx_dtype, dp.w_idx, dp.keys, dp.q_mla, p.q_mla_dtype,
                              dp.latent, L, seq_len, W, max_len, k, p.softmax_scale, ws, indices_out=idx)
        dsa.mla_absorb_out(proj, out, w_uv)
        dsa.dsa_decode_shared(out2, lse2, dp.q_mla, p.q_mla_dtype, dp.latent, L, idx, B, W, p.softmax_scale,
                              workspace=ws2)

    layer()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, idx, proj, out2, lse2)]
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        layer()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (out, lse, proj, out2, lse2):
            t.fill_(float("nan"))
        idx.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "idx", "proj", "shared out", "shared lse"),
                              (out, lse, idx, proj, out2, lse2), ref):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"replay {rep}: {name} differs"
        gpu_decode_step(other)     # unrelated eager work between replays

"""GPU parity of dsa_cache_append against the oracle: after the append every
byte of the key and latent caches, and every fp8 scale, is bit-identical to
the oracle's append of the same tokens (the fp8 code is an integer decided in
float32 on both sides); the appended caches then feed a decode step whose
scores and indices match the oracle on those caches."""
import numpy as np
import pytest
import torch

import sparse_attention_14_amd as dsa

import oracle
from sparse_attention_14_amd import device, inputs

from gpu_util import check_scores, gpu_decode_step

pytestmark = pytest.mark.gpu

S = inputs.small
CASES = {
    "fp8_contig_bf16_in": (S(inputs.DECODE_128K_FP8, name="a1", wid=501, batch=3, seq_len=(50, 3000),
                             tie_fraction=0.0, capacity_pad=16), 1, "bf16"),
    "fp8_paged_f32_in_w4": (S(inputs.DECODE_128K_FP8, name="a2", wid=502, batch=4, seq_len=(3, 2000), paged=True,
                              tie_fraction=0.0), 4, "f32"),
    "bf16_paged_w2": (S(inputs.PAGED_DECODE, name="a3", wid=503, batch=5, seq_len=(1, 700)), 2, "bf16"),
    "f32_tiny": (inputs.TINY_FP32, 1, "f32"),
    "fp8_keys_fp8_latent_paged_w2": (S(inputs.DECODE_128K_FP8_LAT8, name="a4", wid=504, batch=3, seq_len=(10, 1000),
                                       paged=True, tie_fraction=0.0), 2, "bf16"),
}


def _dev_raw(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def _append_on_gpu(dp, nk, kdt, nl, seq, pos, keys=True, latent=True):
    dsa.dsa_cache_append(dp.keys if keys else None, _dev_raw(nk) if keys else None, kdt,
                         dp.latent if latent else None, _dev_raw(nl) if latent else None,
                         torch.from_numpy(pos).cuda(), seq=torch.from_numpy(seq).cuda())
    torch.cuda.synchronize()


def _assert_cache_equal(dc, ref):
    assert np.array_equal(dc.rows.cpu().numpy(), ref.storage.reshape(-1))
    if ref.scale is not None:
        assert np.array_equal(dc.scale.cpu().numpy().view(np.uint32), ref.scale.reshape(-1).view(np.uint32))


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_is_bit_identical_to_the_oracle(name):
    wl, window, kdt = CASES[name]
    p = inputs.make_problem(wl)
    nk, nl, seq, pos = inputs.append_tokens(p, window, kdt)
    print(f"case {name}: {len(pos)} tokens, keys {p.keys.dtype} from {kdt}, paged={p.keys.paged}", flush=True)
    dp = device.upload(p)
    ref_k, ref_l = oracle.cache_append(p.keys, nk, kdt, p.latent, nl, seq, pos)
    _append_on_gpu(dp, nk, kdt, nl, seq, pos)
    _assert_cache_equal(dp.keys, ref_k)
    _assert_cache_equal(dp.latent, ref_l)


def test_append_keys_only_and_latent_only():
    wl, window, kdt = CASES["fp8_paged_f32_in_w4"]
    p = inputs.make_problem(wl)
    nk, nl, seq, pos = inputs.append_tokens(p, window, kdt)
    dp = device.upload(p)
    ref_k, _ = oracle.cache_append(p.keys, nk, kdt, None, None, seq, pos)
    _append_on_gpu(dp, nk, kdt, nl, seq, pos, latent=False)
    _assert_cache_equal(dp.keys, ref_k)
    _assert_cache_equal(dp.latent, p.latent)              # untouched
    dp = device.upload(p)
    _, ref_l = oracle.cache_append(None, None, kdt, p.latent, nl, seq, pos)
    _append_on_gpu(dp, nk, kdt, nl, seq, pos, keys=False)
    _assert_cache_equal(dp.keys, p.keys)
    _assert_cache_equal(dp.latent, ref_l)


def test_append_special_values():
    """Zero rows, subnormal float32 inputs, exact e4m3fn midpoints (a row whose
    largest magnitude is 448 has scale 1, so its values are the quotients
    themselves), signed zeros, wide dynamic range and saturation-adjacent values."""
    D = 128
    rows = []
    rows.append(np.zeros(D))
    rng = np.random.default_rng(0)
    rows.append(rng.choice([-1.0, 1.0], D) * rng.uniform(1e-45, 1e-38, D))        # subnormal float32
    mids = []
    for c in range(0, 0x7E):
        lo, hi = oracle.e4m3fn_to_double(c), oracle.e4m3fn_to_double(c + 1)
        mids.append((lo + hi) / 2)
    mids = np.array(mids)
    r = np.concatenate([[448.0], rng.choice(mids, D - 1)])
    r[1::2] *= -1
    rows.append(r)
    r = np.concatenate([[448.0], (2 * np.arange(8) + 1) * 2.0 ** -10, -((2 * np.arange(8) + 1) * 2.0 ** -10),
                        np.zeros(D - 17)])
    r[-1] = -0.0
    rows.append(r)
    rows.append(np.array([1e4, 1e-3, -2e-7, 3e-30] * (D // 4)))
    rows.append(np.full(D, 1e-38))
    r = rng.normal(0, 1, D)
    r[::7] = -0.0
    rows.append(r)
    rows.append(np.array([447.9, -463.9, 1.0, 0.0] * (D // 4)))
    nk = np.array(rows, dtype=np.float32)
    m = nk.shape[0]
    base = inputs.cache_from_values(np.zeros((2, 40, D), np.float32), "e4m3fn", scale=np.ones((2, 40), np.float32),
                                    paged_block=64, seed=1)
    seq = np.array([i % 2 for i in range(m)], dtype=np.int32)
    pos = np.array([3 + 5 * i for i in range(m)], dtype=np.int32)
    ref_k, _ = oracle.cache_append(base, nk, "f32", None, None, seq, pos)
    dk = device.upload_cache(base)
    torch.cuda.synchronize()
    dsa.dsa_cache_append(dk, torch.from_numpy(nk).cuda(), "f32", None, None, torch.from_numpy(pos).cuda(),
                         seq=torch.from_numpy(seq).cuda())
    torch.cuda.synchronize()
    got = dk.rows.cpu().numpy()
    ref = ref_k.storage.reshape(-1)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}: gpu {got[bad[:8]]} oracle {ref[bad[:8]]}"
    assert np.array_equal(dk.scale.cpu().numpy().view(np.uint32), ref_k.scale.reshape(-1).view(np.uint32))


def test_appended_caches_feed_a_decode_step():
    wl, window, kdt = CASES["fp8_contig_bf16_in"]
    p = inputs.make_problem(wl)
    nk, nl, seq, pos = inputs.append_tokens(p, window, kdt)
    dp = device.upload(p)
    ref_k, ref_l = oracle.cache_append(p.keys, nk, kdt, p.latent, nl, seq, pos)
    _append_on_gpu(dp, nk, kdt, nl, seq, pos)
    out, lse, scores, idx, ws = gpu_decode_step(dp)
    g_scores = scores.cpu().numpy()
    p2 = inputs.Problem(**{**p.__dict__, "keys": ref_k, "latent": ref_l})
    ref = oracle.index_scores(p2.q_idx, p2.q_idx_dtype, p2.w_idx, ref_k, p2.q_seq, p2.q_len)
    check_scores(p2, g_scores, ref)
    ref_idx, _ = oracle.topk(g_scores.astype(np.float64), p2.q_len, p2.topk)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)

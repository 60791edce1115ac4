"""Pins for the oracle's absorbed-MLA GEMMs (query absorption q_nope . W_UK and
output projection o_lat . W_UV; "Self-contained GLM-5 serving stack",
component list: absorbed MLA decode; "GLM on an A100, in Vx", "The model":
one compressed latent row per token serves as key and value).

The defining property is the absorption identity: attending with the absorbed
query over the latent rows and projecting the result by W_UV gives exactly
what explicit attention gives with per-token keys W_UK^T latent and values
W_UV^T latent.  That identity, closed forms (identity and one-hot weights)
and exact scaling pin the two functions."""
import numpy as np

from sparse_attention_14_amd import inputs

BF16_ONE = 0x3F80


def _bf16(x):
    return inputs.encode(np.asarray(x, dtype=np.float32), "bf16")


def _dec(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_absorb_q_identity_and_rope_copy(oracle_mod):
    rng = np.random.default_rng(1)
    n_q, H, dn, L, R = 3, 2, 128, 512, 64
    w = np.zeros((H, dn, L), np.uint16)
    for h in range(H):
        w[h, np.arange(dn), np.arange(dn) + 64 * h] = BF16_ONE        # W_UK[h] = identity into columns 64h..
    qn = _bf16(rng.normal(0, 1, (n_q, H, dn)))
    qr = _bf16(rng.normal(0, 1, (n_q, H, R)))
    out = oracle_mod.mla_absorb_q(qn, qr, "bf16", w)
    assert out.shape == (n_q, H, L + R)
    for h in range(H):
        expect = np.zeros((n_q, L))
        expect[:, 64 * h:64 * h + dn] = _dec(qn[:, h])
        assert np.array_equal(out[:, h, :L], expect)
    assert np.array_equal(out[:, :, L:], _dec(qr))


def test_absorb_q_one_hot_query_picks_a_weight_row(oracle_mod):
    rng = np.random.default_rng(2)
    H, dn, L = 3, 64, 128
    w = _bf16(rng.normal(0, 1, (H, dn, L)))
    qn = np.zeros((2, H, dn), np.uint16)
    qn[0, 1, 5] = BF16_ONE
    qn[1, 2, 63] = 0xC000                                             # -2.0
    out = oracle_mod.mla_absorb_q(qn, None, "bf16", w)
    assert np.array_equal(out[0, 1], _dec(w[1, 5]))
    assert np.array_equal(out[1, 2], -2.0 * _dec(w[2, 63]))
    assert np.all(out[0, [0, 2]] == 0) and np.all(out[1, [0, 1]] == 0)


def test_absorb_out_closed_forms(oracle_mod):
    rng = np.random.default_rng(3)
    H, L, dv = 2, 128, 128
    w = np.zeros((H, L, dv), np.uint16)
    w[:, np.arange(L), np.arange(L)] = BF16_ONE
    o = rng.normal(0, 1, (4, H, L)).astype(np.float32)
    assert np.array_equal(oracle_mod.mla_absorb_out(o, w), o.astype(np.float64))
    w = _bf16(rng.normal(0, 1, (H, L, dv)))
    one = np.zeros((1, H, L), np.float32)
    one[0, 1, 7] = 0.5
    got = oracle_mod.mla_absorb_out(one, w)
    assert np.array_equal(got[0, 1], 0.5 * _dec(w[1, 7])) and np.all(got[0, 0] == 0)
    # exact power-of-two scaling
    assert np.array_equal(oracle_mod.mla_absorb_out(4 * o, w), 4 * oracle_mod.mla_absorb_out(o, w))


def test_absorption_identity_matches_explicit_keys_and_values(oracle_mod):
    """Absorbed path (q_nope . W_UK over latent rows, attention, o_lat . W_UV)
    against explicit attention with keys [W_UK^T c | rope] and values W_UV^T c."""
    rng = np.random.default_rng(4)
    n_q, H, dn, dv, L, R, n = 2, 3, 64, 96, 128, 32, 40
    scale = 1.0 / np.sqrt(dn + R)
    w_uk = _bf16(rng.normal(0, 1 / np.sqrt(L), (H, dn, L)))
    w_uv = _bf16(rng.normal(0, 1 / np.sqrt(L), (H, L, dv)))
    qn = _bf16(rng.normal(0, 1, (n_q, H, dn)))
    qr = _bf16(rng.normal(0, 1, (n_q, H, R)))
    lat = rng.normal(0, 1, (1, n, L + R)).astype(np.float32)
    cache = inputs.cache_from_values(lat, "f32")
    idx = np.tile(np.arange(n, dtype=np.int32), (n_q, 1))
    q_seq = np.zeros(n_q, np.int32)

    q_abs = oracle_mod.mla_absorb_q(qn, qr, "bf16", w_uk)
    o_lat, _, p_abs = oracle_mod.mla_attend(q_abs.astype(np.float32), "f32", cache, L, idx, q_seq, scale,
                                            want_probs=True)
    out_abs = oracle_mod.mla_absorb_out(o_lat.astype(np.float32), w_uv)

    c = lat[0].astype(np.float64)                                    # [n, L + R]
    Wk, Wv = _dec(w_uk), _dec(w_uv)
    for i in range(n_q):
        for h in range(H):
            keys = np.concatenate([c[:, :L] @ Wk[h].T, c[:, L:]], axis=1)    # [n, dn + R]
            q = np.concatenate([_dec(qn[i, h]), _dec(qr[i, h])])
            z = scale * keys @ q
            p = np.exp(z - z.max())
            p /= p.sum()
            vals = c[:, :L] @ Wv[h]                                  # [n, dv]
            explicit = p @ vals
            assert np.allclose(p_abs[i, h, :n], p, rtol=1e-5, atol=1e-9)
            assert np.allclose(out_abs[i, h], explicit, rtol=1e-5, atol=1e-6 * np.abs(explicit).max())

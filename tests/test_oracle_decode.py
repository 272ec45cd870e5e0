"""Pins for the oracle's decode step: exact softmax attention over the valid
slots of the fixed cache (companion page "Prefill / Decode Pipeline" and "Ring
Buffer vs. Naive Slicing")."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import CacheState, Config, decode_step, prefill_compress_one


def _cfg(**kw):
    base = dict(n_q_heads=4, n_kv_heads=2, d_qk=16, d_v=16, L_sink=2, K=3, L_recent=5,
                W=2, pool=3)
    base.update(kw)
    return Config(**base)


def _complex_rope(x, pos, theta, d):
    h = d // 2
    z = x[..., :h] + 1j * x[..., h:]
    z = z * np.exp(1j * pos * theta ** (-2.0 * np.arange(h) / d))
    return np.concatenate([z.real, z.imag], axis=-1)


def _sdpa(q, k, v, scale):
    """library attention, float64 CPU: q [H, d], k/v [H, n, d]"""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    out = F.scaled_dot_product_attention(t(q)[:, None, None, :], t(k)[:, None], t(v)[:, None],
                                         scale=scale)
    return out[:, 0, 0].numpy()


@pytest.mark.parametrize("L", [0, 1, 6])
def test_equals_full_causal_attention_while_below_capacity(L):
    # no compression has happened and n <= C: the fixed cache holds the whole
    # history, so decode is ordinary causal attention over every token
    theta = 1e4
    cfg = _cfg(rope_theta=theta, rope_begin=0, rope_end=16)
    G, C = cfg.G, cfg.C
    rng = np.random.default_rng(L)
    k0 = rng.standard_normal((2, L, 16))
    v0 = rng.standard_normal((2, L, 16))
    state = CacheState(cfg, 1)
    state.admit(0, prefill_compress_one(cfg, rng.standard_normal((4, 2, 16)), k0, v0))
    hist_k, hist_v = [k0[:, t] for t in range(L)], [v0[:, t] for t in range(L)]
    for t in range(L, C):
        q = rng.standard_normal((1, 4, 16))
        kn, vn = rng.standard_normal((1, 2, 16)), rng.standard_normal((1, 2, 16))
        out, err = decode_step(state, q, kn, vn, np.array([t]))
        assert not err
        krot = _complex_rope(kn[0], t, theta, 16).astype(np.float32).astype(np.float64)
        hist_k.append(krot)
        hist_v.append(vn[0])
        K_all = np.stack(hist_k, axis=1)      # [Hkv, t+1, d]
        V_all = np.stack(hist_v, axis=1)
        qr = _complex_rope(q[0], t, theta, 16)
        ref = _sdpa(qr, np.repeat(K_all, G, axis=0), np.repeat(V_all, G, axis=0),
                    cfg.sm_scale)
        np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)


def test_no_middle_segment_is_sliding_window_attention():
    # L_sink = K = 0: the cache is a pure ring over the last L_recent tokens
    cfg = _cfg(L_sink=0, K=0, L_recent=4)
    rng = np.random.default_rng(9)
    state = CacheState(cfg, 1)
    ks, vs = [], []
    for t in range(15):
        q = rng.standard_normal((1, 4, 16))
        kn, vn = rng.standard_normal((1, 2, 16)), rng.standard_normal((1, 2, 16))
        out, _ = decode_step(state, q, kn, vn, np.array([t]))
        ks.append(kn[0].astype(np.float32).astype(np.float64))
        vs.append(vn[0])
        Kw = np.stack(ks[-4:], axis=1)
        Vw = np.stack(vs[-4:], axis=1)
        ref = _sdpa(q[0], np.repeat(Kw, 2, axis=0), np.repeat(Vw, 2, axis=0), cfg.sm_scale)
        np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)


def test_output_does_not_depend_on_slot_order():
    # permuting the sink + middle slots (which the next write never touches)
    # must not change the attention output
    cfg = _cfg()
    rng = np.random.default_rng(4)
    L = 30
    res = prefill_compress_one(cfg, rng.standard_normal((4, 2, 16)),
                               rng.standard_normal((2, L, 16)), rng.standard_normal((2, L, 16)))
    a, b = CacheState(cfg, 1), CacheState(cfg, 1)
    a.admit(0, res)
    b.admit(0, res)
    n = cfg.L_sink + cfg.K
    perm = rng.permutation(n)
    b.k[0, :, :n] = b.k[0][:, perm]
    b.v[0, :, :n] = b.v[0][:, perm]
    b.slot_pos[0, :, :n] = b.slot_pos[0][:, perm]
    for t in range(L, L + 8):
        q = rng.standard_normal((1, 4, 16))
        kn, vn = rng.standard_normal((1, 2, 16)), rng.standard_normal((1, 2, 16))
        out_a, _ = decode_step(a, q, kn, vn, np.array([t]))
        out_b, _ = decode_step(b, q, kn, vn, np.array([t]))
        np.testing.assert_allclose(out_a, out_b, rtol=0, atol=1e-14)


def test_single_valid_slot_returns_its_value():
    cfg = _cfg()
    rng = np.random.default_rng(2)
    state = CacheState(cfg, 2)
    q = rng.standard_normal((2, 4, 16))
    kn, vn = rng.standard_normal((2, 2, 16)), rng.standard_normal((2, 2, 16))
    out, err = decode_step(state, q, kn, vn, np.array([0, -1]))
    assert not err
    for j in range(4):
        np.testing.assert_allclose(out[0, j], vn[0, j // 2], rtol=0, atol=1e-15)
    assert (out[1] == 0).all()                              # inactive row
    assert state.n_tokens[1] == 0 and (state.slot_pos[1] == -1).all()


def test_latent_value_alias_equals_explicit_copy():
    # MLA absorbed form: the value is the first d_v dims of the shared latent
    # key.  With the rotary range outside those dims, an explicit value cache
    # fed the (storage-rounded) latent prefix is ordinary MQA and must agree.
    kw = dict(n_q_heads=8, n_kv_heads=1, d_qk=24, d_v=16, L_sink=2, K=3, L_recent=5, W=2,
              pool=3, rope_theta=1e4, rope_begin=16, rope_end=24)
    mla, mqa = _cfg(v_aliases_k=True, **kw), _cfg(**kw)
    rng = np.random.default_rng(11)
    L = 25
    q0, k0 = rng.standard_normal((8, 2, 24)), rng.standard_normal((1, L, 24))
    sa, sb = CacheState(mla, 1), CacheState(mqa, 1)
    sa.admit(0, prefill_compress_one(mla, q0, k0, None))
    sb.admit(0, prefill_compress_one(mqa, q0, k0, k0[..., :16].copy()))
    for t in range(L, L + 12):
        q, kn = rng.standard_normal((1, 8, 24)), rng.standard_normal((1, 1, 24))
        vn = kn[..., :16].astype(np.float32).astype(np.float64)
        oa, _ = decode_step(sa, q, kn, None, np.array([t]))
        ob, _ = decode_step(sb, q, kn, vn, np.array([t]))
        np.testing.assert_array_equal(oa, ob)


def test_position_mismatch_sets_error_and_applies_step_at_pos():
    cfg = _cfg()
    rng = np.random.default_rng(1)
    state = CacheState(cfg, 1)
    _, err = decode_step(state, rng.standard_normal((1, 4, 16)), rng.standard_normal((1, 2, 16)),
                         rng.standard_normal((1, 2, 16)), np.array([3]))
    assert err and state.n_tokens[0] == 4 and (state.slot_pos[0, :, 3] == 3).all()


def test_decode_write_updates_only_the_ring_slot():
    # the write half of a step: the rotated key rounded to bf16 in slot
    # ring_slot(pos), the value copied, slot_pos and n_tokens advanced; an
    # inactive row and every other slot untouched; a stale pos is flagged
    from oracle import decode_write, ring_slot, rope_rotate, round_to_bf16
    cfg = Config(n_q_heads=2, n_kv_heads=1, d_qk=4, d_v=4, L_sink=1, K=2, L_recent=3, W=1,
                 pool=1, rope_theta=1e4, rope_begin=0, rope_end=4, dtype="bf16")
    st = CacheState(cfg, 2)
    rng = np.random.default_rng(3)
    st.k[:] = round_to_bf16(rng.standard_normal(st.k.shape))
    st.v[:] = round_to_bf16(rng.standard_normal(st.v.shape))
    st.n_tokens[:] = [9, 4]
    before_k, before_v = st.k.copy(), st.v.copy()
    kn = round_to_bf16(rng.standard_normal((2, 1, 4)))
    vn = round_to_bf16(rng.standard_normal((2, 1, 4)))
    err = decode_write(st, kn, vn, np.array([9, -1]))
    assert not err
    slot = 1 + 2 + (9 - 3) % 3
    assert slot == ring_slot(9, 1, 2, 3) == 3
    np.testing.assert_array_equal(st.k[0, 0, slot], round_to_bf16(rope_rotate(kn[0], 9, 1e4, 0, 4))[0])
    np.testing.assert_array_equal(st.v[0, 0, slot], vn[0, 0])
    others = [s for s in range(cfg.C) if s != slot]
    np.testing.assert_array_equal(st.k[0, :, others], before_k[0, :, others])
    np.testing.assert_array_equal(st.k[1], before_k[1])
    np.testing.assert_array_equal(st.v[1], before_v[1])
    assert list(st.n_tokens) == [10, 4] and st.slot_pos[0, 0, slot] == 9
    assert decode_write(st, kn, vn, np.array([12, -1]))   # n_tokens is 10: stale

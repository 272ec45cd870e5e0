"""GPU parity of ss_decode_step against the fp64 oracle.

Both sides start from the oracle's prefill state (uploaded bit-exactly), then
take the same seeded decode inputs step by step; one full-shape test instead
decodes from the library's own prefill (see there).  Checked every step: the
attention output (max-abs <= 1e-4 fp32, <= 2e-2 bf16), the written slot of
every row (slot_pos exact, rotated key and value bit-exact), n_tokens."""
import numpy as np
import pytest
import torch

from kv_cache_compression_obs_amd import snapstream as ss
from kv_cache_compression_obs_amd import synth
from parity import OUT_TOL, decode_case, lib_config, say

pytestmark = pytest.mark.gpu


def test_decode_tiny_fp32_after_compression():
    w = synth.workload("tiny_fp32")
    say("decode tiny_fp32 L=512 steps=64")
    decode_case(w, L=512, steps=64, seed=1)


def test_decode_tiny_fp32_ring_wraps():
    w = synth.workload("tiny_fp32")
    say("decode tiny_fp32 L=512 steps=300 (ring index wraps)")
    decode_case(w, L=512, steps=300, seed=2, check_every=7)


def test_decode_tiny_fp32_short_prompt_crosses_capacity():
    # uncompressed prompt of 100 tokens; the valid prefix grows through n = C
    w = synth.workload("tiny_fp32")
    say("decode tiny_fp32 L=100 steps=160")
    decode_case(w, L=100, steps=160, seed=3, check_every=3)


def test_decode_empty_prompt_single_slot():
    w = synth.workload("tiny_fp32")
    say("decode tiny_fp32 L=1 steps=3")
    decode_case(w, L=1, steps=3, seed=4)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_bf16_rope_ring(d):
    w = synth.workload("llama8b_c4k", B=3, d_qk=d, d_v=d, rope_end=d, L_sink=4, K=28,
                       L_recent=64)
    say(f"decode bf16 d={d} C=96 L=200 steps=150")
    decode_case(w, L=200, steps=150, seed=5, check_every=5)


@pytest.mark.parametrize("rope", [(32, 96), (2, 66), (0, 0)],
                         ids=["aligned_partial", "unaligned", "none"])
def test_decode_bf16_rope_ranges(rope):
    # bf16 caches decode through the direct-load ring kernel when the rotary
    # range starts and splits on multiples of 8 dims (or is empty); other
    # ranges take the register-tile kernel.  Both must match the oracle.
    b, e = rope
    w = synth.workload("llama8b_c4k", B=2, rope_begin=b, rope_end=e,
                       rope_theta=500000.0 if e > b else 0.0, L_sink=4, K=28, L_recent=64)
    say(f"decode bf16 rope [{b}, {e}) C=96 L=200 steps=40")
    decode_case(w, L=200, steps=40, seed=11, check_every=3)


@pytest.mark.parametrize("g", [1, 16])
def test_decode_bf16_group_sizes(g):
    # one q-head per kv-head, and the largest group (16 q-heads)
    w = synth.workload("llama8b_c4k", B=2, n_q_heads=2 * g, n_kv_heads=2, W=16, L_sink=4,
                       K=60, L_recent=200)
    say(f"decode bf16 G={g} C=264 L=500 steps=30")
    decode_case(w, L=500, steps=30, seed=12, check_every=4)


def test_decode_bf16_mixed_rows_inactive_and_mismatch():
    # the mixed-rows case on bf16 caches: an inactive row (pos < 0), a row
    # whose pos jumps ahead of n_tokens once (error flag, step applied at
    # pos), every row crossing C = 96 during the run
    w = synth.workload("llama8b_c4k", B=4, L_sink=4, K=28, L_recent=64)
    L = 90
    base = np.array([L, L, L, L])

    def positions(t):
        p = base + t
        if t < 4:
            p[2] = -1
        else:
            p[2] = L + t - 4
        if t >= 6:
            p[3] = L + t + 2
        return p

    say("decode bf16 mixed rows C=96")
    decode_case(w, L=L, steps=14, seed=13, positions=positions)


def test_decode_fp32_d128_rope():
    w = synth.workload("llama8b_c4k", B=2, dtype="f32", L_sink=4, K=28, L_recent=64)
    say("decode f32 d=128 C=96 L=300 steps=70")
    decode_case(w, L=300, steps=70, seed=6, check_every=3)


def test_decode_mixed_rows_inactive_and_mismatch():
    # continuous batching: rows at different points of their life; row 2 is
    # inactive (pos < 0) for a while; row 3 gives pos != n_tokens once (error
    # flag, step applied at pos)
    w = synth.workload("tiny_fp32", B=4)
    L = 150
    base = np.array([L, L, L, L])

    def positions(t):
        p = base + t
        if t < 5:
            p[2] = -1
        elif t >= 5:
            p[2] = L + t - 5
        if t == 9:
            p[3] = L + t + 3
        elif t > 9:
            p[3] = L + t + 3
        return p

    say("decode mixed rows")
    decode_case(w, L=L, steps=20, seed=7, positions=positions)


def test_decode_llama8b_c4k_full_shape():
    # 16 rows x 8 kv-heads x C=4096 (bf16, rope 5e5): the benchmark's decode
    # launch configuration; oracle compares every output of 3 steps
    w = synth.workload("llama8b_c4k")
    say("decode llama8b_c4k full B=16 L=16384 steps=3")
    worst = decode_case(w, L=w["L"], steps=3, seed=8)
    say(f"  worst max-abs {worst:.3g}")


def test_decode_uncompressed_128k_cache():
    # the uncompressed baseline's shape: a cache of C = L = 131072 slots that
    # holds the whole prompt as it is (no scoring), every slot valid; the
    # decode steps evict from the start of the recent window
    w = synth.workload("llama8b_128k", B=2, L_recent=131072 - 64 - 960)
    say("decode uncompressed C=L=131072 B=2 steps=2")
    worst = decode_case(w, L=131072, steps=2, seed=10)
    say(f"  worst max-abs {worst:.3g}")


def test_decode_is_deterministic_and_workspace_reusable():
    # same inputs on two copies of the cache give bitwise-identical outputs
    # (fixed split order), and a workspace reused for many calls stays valid
    w = synth.workload("llama8b_c4k", B=4, L_sink=16, K=240, L_recent=256)
    cfg = lib_config(w)
    inp = synth.prefill_inputs(w, 9, device="cuda", L=2000)
    cache = ss.Cache(cfg, 4)
    ss.ss_prefill_compress(cfg, inp["q_obs"], inp["k"], inp["v"], cache)
    twin = cache.clone()
    dec = synth.decode_inputs(w, 9, 12, device="cuda", B=4)
    ws = ss.decode_workspace(cfg, 4)
    outs = []
    for c in (cache, twin):
        o = torch.empty(4, 32, 128, dtype=torch.bfloat16, device="cuda")
        got = []
        for t in range(12):
            pos = torch.full((4,), 2000 + t, dtype=torch.int32, device="cuda")
            ss.ss_decode_step(cfg, dec["q"][t], dec["k_new"][t], dec["v_new"][t], pos, c, o, ws=ws)
            got.append(o.clone())
        outs.append(torch.stack(got))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(cache.k, twin.k) and torch.equal(cache.v, twin.v)
    assert torch.equal(cache.slot_pos, twin.slot_pos)
    counters = ws[:4 * 8 * 4].view(torch.int32)
    assert int(counters.abs().sum().item()) == 0


def test_decode_from_library_prefill_llama8b_c4k():
    # the library's own prefill-then-decode chain at full shape (16 x 8
    # groups, 16384 -> 4096 slots): nothing is uploaded from the oracle.  Two
    # requests are followed: their selections are checked against the oracle
    # under the tie-band rule, their cache rows must be bit-exact copies of the
    # layout of the validated selection, and every one of 24 decode steps is
    # compared (outputs, written slot, token count)
    import oracle
    from parity import compare_selection, oracle_config, oracle_prefill_request
    w = synth.workload("llama8b_c4k")
    B, C, H = w["B"], w["C"], w["n_kv_heads"]
    cfg = lib_config(w)
    inp = synth.prefill_inputs(w, 81, device="cuda")
    cache = ss.Cache(cfg, B)
    sel = torch.full((B, H, w["K"]), -1, dtype=torch.int32, device="cuda")
    ss.ss_prefill_compress(cfg, inp["q_obs"], inp["k"], inp["v"], cache, sel_out=sel)
    follow = [3, 12]
    state = oracle.CacheState(oracle_config(w), len(follow))
    for i, bi in enumerate(follow):
        res = oracle_prefill_request(w, inp, bi)
        sel_lib = sel[bi].cpu().numpy().astype(np.int64)
        for h in range(H):
            compare_selection(sel_lib[h], res.pooled[h], res.sel[h], w["K"])
        k_c, v_c, sp = oracle.fixed_cache_layout(oracle_config(w), synth.to_f64(inp["k"][bi]),
                                                 synth.to_f64(inp["v"][bi]), sel_lib)
        np.testing.assert_array_equal(cache.slot_pos[bi].cpu().numpy(), sp)
        assert np.array_equal(cache.k[bi].double().cpu().numpy(), k_c)
        assert np.array_equal(cache.v[bi].double().cpu().numpy(), v_c)
        state.k[i], state.v[i], state.slot_pos[i], state.n_tokens[i] = k_c, v_c, sp, w["L"]
    steps = 24
    dec = synth.decode_inputs(w, 81, steps, device="cuda")
    out = torch.empty(B, w["n_q_heads"], w["d_v"], dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = ss.decode_workspace(cfg, B)
    fidx = torch.tensor(follow, device="cuda")
    worst = 0.0
    for t in range(steps):
        p = w["L"] + t
        ss.ss_decode_step(cfg, dec["q"][t], dec["k_new"][t], dec["v_new"][t],
                          torch.full((B,), p, dtype=torch.int32, device="cuda"), cache, out, err,
                          ws)
        ref, ref_err = oracle.decode_step(state, synth.to_f64(dec["q"][t][fidx]),
                                          synth.to_f64(dec["k_new"][t][fidx]),
                                          synth.to_f64(dec["v_new"][t][fidx]), np.full(2, p))
        torch.cuda.synchronize()
        diff = np.abs(out[fidx].double().cpu().numpy() - ref).max()
        worst = max(worst, diff)
        assert diff <= OUT_TOL["bf16"], f"step {t}: max-abs {diff:.3g}"
        slot = oracle.ring_slot(p, w["L_sink"], w["K"], w["L_recent"])
        for i, bi in enumerate(follow):
            np.testing.assert_array_equal(cache.k[bi, :, slot].double().cpu().numpy(),
                                          state.k[i, :, slot])
        assert not ref_err
    assert int(err.item()) == 0
    assert np.all(cache.n_tokens.cpu().numpy() == w["L"] + steps)
    say(f"  decode from the library's prefill: worst max-abs {worst:.3g}")

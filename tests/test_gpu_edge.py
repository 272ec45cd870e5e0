"""GPU parity on the degenerate and boundary configurations of the method:
no middle budget (K = 0), no sinks (L_sink = 0), no pooling (pool = 1), a
one-query observation window (W = 1), plain multi-head attention (G = 1), the
largest group the score kernels take (G = 16, G*W = 256 rows), rotary
embedding over part of the head (decode rotates dims 32..95 of 128) or over
every dim of an fp32 head, and pooling windows at and past the select
kernel's LDS staging limit (also on a group long enough for the select to be
split over several workgroups) or wider than the whole middle region, middle
regions of 201 and 17 keys on the 128-row score kernels, and a batch of 2048
rows.  Each
configuration runs the prefill comparison (scores, selection, slot map,
gathered rows) and a decode run across the ring wrap (outputs, written rows,
n_tokens) against the oracle."""
import pytest

from kv_cache_compression_obs_amd import synth
from parity import decode_case, prefill_case, say

pytestmark = pytest.mark.gpu

TINY = "tiny_fp32"          # 4q/2kv, d64, fp32, S/K/R = 4/64/128, W 16, pool 7
SMALL = "llama8b_c4k"       # 32q/8kv, d128, bf16, rope 5e5

CASES = {
    "no_middle_budget": (TINY, dict(K=0), 512),
    "no_sinks": (TINY, dict(L_sink=0), 512),
    "no_pooling": (TINY, dict(pool=1), 512),
    "one_query_window": (TINY, dict(W=1), 512),
    "multi_head_G1": (TINY, dict(n_q_heads=2, n_kv_heads=2), 512),
    "fp32_full_rope": (TINY, dict(rope_theta=1e4, rope_begin=0, rope_end=64), 512),
    "largest_group_G16": (SMALL, dict(B=2, n_q_heads=32, n_kv_heads=2, W=16, L_sink=16, K=200,
                                      L_recent=512), 3000),
    "partial_rope": (SMALL, dict(B=2, rope_begin=32, rope_end=96, L_sink=16, K=200,
                                 L_recent=512), 3000),
    # pooling half-width at the LDS-staged limit (256) and past it (the select
    # kernel then pools straight from the raw scores); a window wider than the
    # middle region makes every pooled score the maximum (all ties)
    "pool_513_staged_limit": (SMALL, dict(B=2, pool=513, L_sink=16, K=200, L_recent=512), 3000),
    "pool_515_unstaged": (SMALL, dict(B=2, pool=515, L_sink=16, K=200, L_recent=512), 3000),
    "pool_wider_than_middle": (TINY, dict(pool=801), 512),
    # a wide batch: 2048 rows of a 64-slot cache (grids 2048 deep in the
    # row dimension, one short split per row)
    "wide_batch_2048_rows": (TINY, dict(B=2048, L_sink=4, K=16, L_recent=44), 100),
    # short middle regions on the 128-row bf16 score kernels: 201 middle
    # keys (a ragged last tile; each wave owns fewer tiles than its ring
    # holds) and 17 (one full tile and a one-key tile: two waves own no tile)
    "middle_201_keys": (SMALL, dict(B=2, L_sink=16, K=200, L_recent=512), 729),
    "middle_17_keys": (SMALL, dict(B=2, L_sink=16, K=10, L_recent=512), 545),
    # 39472 middle keys: the select work is split over parts of the group,
    # and the 515-wide window is pooled straight from the raw scores
    "pool_515_split_select": (SMALL, dict(B=1, n_q_heads=8, n_kv_heads=2, pool=515, L_sink=16,
                                          K=3000, L_recent=512), 40000),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_edge_prefill(case):
    name, kw, L = CASES[case]
    prefill_case(synth.workload(name, **kw), 61, L=L)


@pytest.mark.parametrize("case", sorted(CASES))
def test_edge_decode(case):
    name, kw, L = CASES[case]
    w = synth.workload(name, **kw)
    steps = w["L_recent"] + 40  # every ring slot rewritten at least once
    say(f"decode edge {case} C={w['C']} L={L} steps={steps}")
    decode_case(w, L=L, steps=steps, seed=62, check_every=max(1, steps // 25))


def test_edge_prefill_all_ties_multi_chunk():
    # zero observation queries: every visible key gets the same probability
    # in every row, so every middle score (and every pooled score) is equal
    # and the selection must be the K lowest middle indices.  39472 middle
    # keys: the select kernel pools them in three LDS-staged chunks (halos at
    # the chunk seams) and re-reads the pooled scores from memory for its
    # radix passes and the compaction.
    import numpy as np
    from parity import check_prefill_group, run_lib_prefill
    w = synth.workload(SMALL, B=1, n_q_heads=8, n_kv_heads=2, L_sink=16, K=3000, L_recent=512)
    L = 40000
    say(f"prefill all ties L={L} m={L - 16 - 512}")
    inp = synth.prefill_inputs(w, 63, device="cuda", L=L)
    inp["q_obs"].zero_()
    res = run_lib_prefill(w, inp)
    cache, raw, pooled, sel = res
    for h in range(2):
        assert (sel[0, h] == np.arange(3000)).all()
        assert np.all(pooled[0, h] == pooled[0, h, 0])
        check_prefill_group(w, inp, res, 0, h)


def test_binding_rejects_tensors_of_the_wrong_shape():
    # the kernels index every tensor by the shape the config implies; the
    # binding refuses a smaller tensor before anything is launched
    import torch

    from kv_cache_compression_obs_amd import snapstream as ss
    w = synth.workload(SMALL, B=4, L_sink=16, K=200, L_recent=512)
    cfg = ss.make_config(**w)
    cache = ss.Cache(cfg, 4)
    q = torch.zeros(4, 32, 128, dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros(4, 8, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(4, 32, 128, dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(4, dtype=torch.int32, device="cuda")
    for bad in (dict(pos=pos[:3]), dict(q=q[:, :16].contiguous()), dict(out=out[:2]),
                dict(kn=kn[..., :64].contiguous())):
        a = dict(q=q, kn=kn, out=out, pos=pos)
        a.update(bad)
        with pytest.raises(ValueError):
            ss.ss_decode_step(cfg, a["q"], a["kn"], a["kn"], a["pos"], cache, a["out"])
    inp = synth.prefill_inputs(w, 5, device="cuda", B=2, L=1000)
    with pytest.raises(ValueError):                       # window of the wrong length
        ss.ss_prefill_compress(cfg, inp["q_obs"][:, :, :16].contiguous(), inp["k"], inp["v"], cache)
    with pytest.raises(ValueError):                       # sel_out too short
        ss.ss_prefill_compress(cfg, inp["q_obs"], inp["k"], inp["v"], cache,
                               sel_out=torch.zeros(2, 8, 10, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int(cache.n_tokens.sum().item()) == 0

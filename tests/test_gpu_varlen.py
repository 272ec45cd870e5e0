"""GPU parity of ss_prefill_compress_varlen: prompts of different lengths
(some stored as they are, some compressed) packed per kv-head and built into
their cache rows by one call.  Every request is checked against the oracle
exactly as a single-request prefill of its own tokens: scores, pooled scores,
selection (tie-band rule), slot maps, bit-exact cache rows, n_tokens."""
import numpy as np
import pytest
import torch

from kv_cache_compression_obs_amd import snapstream as ss
from kv_cache_compression_obs_amd import synth
from parity import check_prefill_group, lib_config, lse_obs, say

pytestmark = pytest.mark.gpu


def _varlen_case(w, seed, lens, rows=None, given_lse=False, max_L=None, B_max=None):
    b, Hkv, C = len(lens), w["n_kv_heads"], w["C"]
    S, R, K = w["L_sink"], w["L_recent"], w["K"]
    max_L = max_L or max(lens)
    say(f"varlen {w['name']} d={w['d_qk']} lengths {lens} (C={C}, max_L={max_L})"
        + (" given lse" if given_lse else ""))
    reqs = [synth.prefill_inputs(w, seed * 1000 + i, device="cuda", B=1, L=n)
            for i, n in enumerate(lens)]
    q_obs = torch.cat([r["q_obs"] for r in reqs]).contiguous()
    k = torch.cat([r["k"][0] for r in reqs], dim=1).contiguous()          # [Hkv, T, d]
    v = (torch.cat([r["v"][0] for r in reqs], dim=1).contiguous()
         if reqs[0]["v"] is not None else None)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    m_max = max(max_L - S - R, 1)
    raw = torch.full((b, Hkv, m_max), float("nan"), device="cuda")
    pooled = torch.full((b, Hkv, m_max), float("nan"), device="cuda")
    sel = torch.full((b, Hkv, max(K, 1)), -7, dtype=torch.int32, device="cuda")[..., :K].contiguous()
    lse = None
    if given_lse:
        lse = torch.zeros(b, w["n_q_heads"], w["W"], dtype=torch.float32, device="cuda")
        for i, r in enumerate(reqs):
            if lens[i] > C:
                lse[i] = lse_obs(w, r)[0]
    cfg = lib_config(w)
    cache = ss.Cache(cfg, B_max or b)
    rows_t = torch.tensor(rows, dtype=torch.int32, device="cuda") if rows else None
    ss.ss_prefill_compress_varlen(cfg, q_obs, k, v, cu, max_L, cache, rows=rows_t, lse=lse,
                                  raw_out=raw, pooled_out=pooled, sel_out=sel)
    torch.cuda.synchronize()
    raw, pooled, sel = raw.cpu().numpy(), pooled.cpu().numpy(), sel.cpu().numpy()
    for i, n in enumerate(lens):
        row = rows[i] if rows else i
        if n > max_L:   # longer than the bound: stored as an empty request
            assert (cache.slot_pos[row] == -1).all() and int(cache.n_tokens[row].item()) == 0
            continue
        m = n - S - R
        res = ((cache, raw[i:i + 1, :, :m], pooled[i:i + 1, :, :m], sel[i:i + 1]) if n > C
               else (cache, None, None, None))
        for h in range(Hkv):
            check_prefill_group(w, reqs[i], res, 0, h, row=row)


def test_varlen_tiny_fp32_mixed():
    # C = 196: 512, 197 and 300 are compressed; 100, 196 and 1 stored as they are
    _varlen_case(synth.workload("tiny_fp32"), 51, [512, 100, 196, 197, 300, 1])


@pytest.mark.parametrize("given_lse", [False, True])
def test_varlen_bf16_d128_into_chosen_rows(given_lse):
    w = synth.workload("llama8b_c4k", L_sink=16, K=200, L_recent=512)   # C = 728
    _varlen_case(w, 52, [4999, 700, 728, 729, 2048, 64, 3000], rows=[7, 0, 5, 2, 6, 1, 3],
                 given_lse=given_lse, B_max=8)


def test_varlen_mla_latent():
    w = synth.workload("deepseek_mla_128k", L_sink=16, K=200, L_recent=512)
    _varlen_case(w, 53, [3000, 500, 1500])


def test_varlen_request_longer_than_bound_is_stored_empty():
    # max_L = 400 but request 1 has 512 tokens: that row is left empty, the
    # others are built as usual
    _varlen_case(synth.workload("tiny_fp32"), 54, [300, 512, 150], max_L=400)


def test_varlen_long_requests_split_select():
    # the longest request has 19472 middle keys, past the select kernel's
    # one-workgroup limit (16384): every group is selected in parts of 3904
    # keys (5 parts), so the 5000-token request has empty parts and the
    # 700-token one (C = 728) is stored as it is
    w = synth.workload("llama8b_c4k", L_sink=16, K=200, L_recent=512)
    _varlen_case(w, 55, [20000, 700, 5000, 18000])

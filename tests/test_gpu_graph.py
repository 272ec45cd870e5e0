"""Both library calls enqueue only kernels on the caller's stream (no
allocation, no memset, no host synchronisation), so they can be captured into
a HIP graph: for bf16 heads of 128 dims, fp32 heads of 64 dims and latent
rows (each decode kernel and each family of score passes).  Each test
captures the calls once, then replays the graph three times; between replays the program does its own eager work (restoring the
cache, poisoning the outputs) and synchronises, and every replay must match
the eager run bit for bit (the kernels are deterministic).  The library keeps
no global state either: decode on two streams at once, each with its own
workspace, gives the sequential results."""
import pytest
import torch

from kv_cache_compression_obs_amd import snapstream as ss
from kv_cache_compression_obs_amd import synth
from parity import lib_config, say

pytestmark = pytest.mark.gpu

W = dict(B=4, L_sink=16, K=200, L_recent=512)  # llama8b_c4k shapes, C = 728
# the three decode kernels and both families of score passes: bf16 heads of
# 128 dims (ring decode), fp32 heads of 64 dims, latent rows
GRAPH_CASES = {
    "llama8b_c4k": (dict(W), 2000, 3000),
    "tiny_fp32": (dict(B=4), 512, 512),
    "deepseek_mla_128k": (dict(W), 2000, 3000),
}


def _restore(dst: ss.Cache, src: ss.Cache):
    dst.k.copy_(src.k)
    if dst.v is not None:
        dst.v.copy_(src.v)
    dst.slot_pos.copy_(src.slot_pos)
    dst.n_tokens.copy_(src.n_tokens)


def _same_cache(a: ss.Cache, b: ss.Cache):
    assert torch.equal(a.k, b.k) and (a.v is None or torch.equal(a.v, b.v))
    assert torch.equal(a.slot_pos, b.slot_pos) and torch.equal(a.n_tokens, b.n_tokens)


@pytest.mark.parametrize("name", sorted(GRAPH_CASES))
def test_decode_steps_replay_in_a_graph(name):
    kw, L, _ = GRAPH_CASES[name]
    w = synth.workload(name, **kw)
    cfg = lib_config(w)
    B, T = w["B"], 4
    say(f"graph decode {name}: {T} steps, B={B}, C={w['C']}")
    inp = synth.prefill_inputs(w, 70, device="cuda", L=L)
    base = ss.Cache(cfg, B)
    ss.ss_prefill_compress(cfg, inp["q_obs"], inp["k"], inp["v"], base)
    dec = synth.decode_inputs(w, 71, T, device="cuda")
    pos = [torch.full((B,), L + t, dtype=torch.int32, device="cuda") for t in range(T)]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = ss.decode_workspace(cfg, B)
    shape = (B, w["n_q_heads"], w["d_v"])
    dt = synth.TORCH_DTYPE[w["dtype"]]

    ref = base.clone()
    ref_out = [torch.empty(shape, dtype=dt, device="cuda") for _ in range(T)]
    vn = [dec["v_new"][t] if dec["v_new"] is not None else None for t in range(T)]
    for t in range(T):
        ss.ss_decode_step(cfg, dec["q"][t], dec["k_new"][t], vn[t], pos[t], ref, ref_out[t], err,
                          ws=ws)
    torch.cuda.synchronize()

    cache = base.clone()
    out = [torch.empty(shape, dtype=dt, device="cuda") for _ in range(T)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(T):
            ss.ss_decode_step(cfg, dec["q"][t], dec["k_new"][t], vn[t], pos[t], cache, out[t],
                              err, ws=ws)
    for rep in range(3):
        _restore(cache, base)
        for o in out:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t in range(T):
            assert torch.equal(out[t], ref_out[t]), f"replay {rep}, step {t}"
        _same_cache(cache, ref)
    assert int(err.item()) == 0


@pytest.mark.parametrize("name", sorted(GRAPH_CASES))
def test_prefill_replays_in_a_graph(name):
    kw, _, L = GRAPH_CASES[name]
    w = synth.workload(name, **kw)
    cfg = lib_config(w)
    B = w["B"]
    say(f"graph prefill {name}: B={B}, L={L}, C={w['C']}")
    inp = synth.prefill_inputs(w, 72, device="cuda", L=L)
    ws = torch.empty(ss.ss_prefill_workspace_bytes(cfg, B, L), dtype=torch.uint8, device="cuda")
    sel = torch.empty(B, w["n_kv_heads"], w["K"], dtype=torch.int32, device="cuda")
    ref_sel = torch.empty_like(sel)

    ref = ss.Cache(cfg, B)
    ss.ss_prefill_compress(cfg, inp["q_obs"], inp["k"], inp["v"], ref, sel_out=ref_sel, ws=ws)
    torch.cuda.synchronize()

    empty = ss.Cache(cfg, B)
    cache = ss.Cache(cfg, B)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ss.ss_prefill_compress(cfg, inp["q_obs"], inp["k"], inp["v"], cache, sel_out=sel, ws=ws)
    for rep in range(3):
        _restore(cache, empty)
        sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, ref_sel), f"replay {rep}"
        _same_cache(cache, ref)


def test_decode_on_two_streams_with_separate_workspaces():
    # the library keeps no global state: two streams (default priority)
    # decoding different caches with their own workspaces at the same time
    # give the sequential results
    w = synth.workload("llama8b_c4k", **W)
    cfg = lib_config(w)
    B, L, T = w["B"], 2000, 8
    say(f"two streams: {T} steps each, B={B}")
    caches, decs, wss, errs = [], [], [], []
    for i in range(2):
        inp = synth.prefill_inputs(w, 80 + i, device="cuda", L=L)
        c = ss.Cache(cfg, B)
        ss.ss_prefill_compress(cfg, inp["q_obs"], inp["k"], inp["v"], c)
        caches.append(c)
        decs.append(synth.decode_inputs(w, 90 + i, T, device="cuda"))
        wss.append(ss.decode_workspace(cfg, B))
        errs.append(torch.zeros(1, dtype=torch.int32, device="cuda"))
    pos = [torch.full((B,), L + t, dtype=torch.int32, device="cuda") for t in range(T)]
    shape = (B, w["n_q_heads"], w["d_v"])
    dt = synth.TORCH_DTYPE[w["dtype"]]
    torch.cuda.synchronize()

    def run(i, cache, out):
        d = decs[i]
        for t in range(T):
            ss.ss_decode_step(cfg, d["q"][t], d["k_new"][t], d["v_new"][t], pos[t], cache, out[t],
                              errs[i], ws=wss[i])

    refs = [c.clone() for c in caches]
    ref_out = [[torch.empty(shape, dtype=dt, device="cuda") for _ in range(T)] for _ in range(2)]
    for i in range(2):
        run(i, refs[i], ref_out[i])
    torch.cuda.synchronize()

    out = [[torch.empty(shape, dtype=dt, device="cuda") for _ in range(T)] for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for i, s in enumerate(streams):
        with torch.cuda.stream(s):
            run(i, caches[i], out[i])
    torch.cuda.synchronize()
    for i in range(2):
        for t in range(T):
            assert torch.equal(out[i][t], ref_out[i][t]), f"stream {i}, step {t}"
        _same_cache(caches[i], refs[i])
        assert int(errs[i].item()) == 0

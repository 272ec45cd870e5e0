#!/usr/bin/env python3
"""Benchmark of the SnapStream hot path on one MI355X.

One step = one ss_prefill_compress of the whole batch (one layer) followed by
the workload's decode steps (ss_decode_step), all inputs already resident in
HBM.  Default workload: one tensor-parallel rank's share of a DeepSeek-R1 MLA
layer in absorbed form (8 of 128 q-heads over one shared 576-dim latent whose
first 512 dims are the value), bf16, batch 32, 131072-token prompts
compressed to C = 32768 (64 + 960 + 31744), W = 32, pool 7, RoPE 1e4 on the
latent's last 64 dims, 512 decode steps; the model has 61 such layers.  The
Llama-3.1-8B-shaped layers (16384 -> 4096 at batch 16; 131072 -> 32768 at
batch 8) are measured the same way after the timed steps and reported under
`other_workloads`; the continuous-batching mix (64 rows, C = 32768, 1000
decode steps with four 65536-token admissions) under `continuous_batching`.
Each of these, and the uncompressed-cache baseline, runs in a fresh child
process (`--leg`): buffers allocated after others were freed in the same
process decoded about 5% slower.

Decode runs over `--replicas` distinct copies of the layer's cache in turn
(step t uses copy t mod replicas), so consecutive decode steps do not find
the previous step's cache in the 256 MB Infinity Cache; each copy keeps its
own sequence position.

Prints one JSON line.  `value` = algorithmic HBM bytes of the step (prefill:
prompt keys read once + C cache rows gathered, read and written; decode: every
valid cache row read) per second of wall time.  `roofline` prices the decode
kernel: its average launch duration is the time between a HIP event recorded
right before the step's first decode kernel and one right after its last,
divided by the number of launches (so it includes the short gaps between
back-to-back launches; no marker sits between them).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn HBM GB/s + tokens/s over fixed cache; prefill compress ms/layer"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


class HipEvents:
    """Raw hipEvent_t handles (plumbing for the library's timed entry points)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


def host_info():
    """CPU model, NumPy version and the BLAS library NumPy calls."""
    import platform

    import numpy as np
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                blas.append(f"{p.get('internal_api')} {p.get('version')} "
                            f"({p.get('num_threads')} threads)")
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "numpy": np.__version__, "blas": "; ".join(blas) or "unknown",
            "host_cpus_visible": len(os.sched_getaffinity(0))}


def algorithmic_bytes(w, elem):
    B, Hkv, d, dv, L, C = w["B"], w["n_kv_heads"], w["d_qk"], w["d_v"], w["L"], w["C"]
    row = (d + (0 if w["v_aliases_k"] else dv)) * elem
    decode = B * Hkv * min(L, C) * row                       # every valid slot read once
    prefill = B * Hkv * L * d * elem + 2 * B * Hkv * min(L, C) * row
    return prefill, decode


def score_flops(w):
    """Q_obs.K^T flops of the two score passes per layer: pass 1 over all L
    keys, pass 2 over the m middle keys (algorithmic = pass 1 only)."""
    B, Hq, d, W, L = w["B"], w["n_q_heads"], w["d_qk"], w["W"], w["L"]
    m = L - w["L_sink"] - w["L_recent"]
    rows = B * Hq * W
    return 2.0 * rows * d * L, 2.0 * rows * d * (L + m)


def score_key_bytes(w, elem):
    """Prompt-key bytes the two score passes read (pass 1 all L keys, pass 2
    the m middle keys)."""
    m = w["L"] - w["L_sink"] - w["L_recent"]
    return w["B"] * w["n_kv_heads"] * (w["L"] + m) * w["d_qk"] * elem


def decode_kernel_name(w):
    """The kernel the library runs for this workload's decode step: the
    latent kernel for MLA, the direct-load ring kernel for bf16 K/V caches
    whose rotary range is empty or starts and splits on multiples of 8 dims,
    the register-tile kernel otherwise."""
    if w["v_aliases_k"]:
        return "decode_mla_kernel"
    half = (w["rope_end"] - w["rope_begin"]) // 2 if w["rope_theta"] > 0 else 0
    aligned = half == 0 or (w["rope_begin"] % 8 == 0 and half % 8 == 0)
    if w["dtype"] == "bf16" and w["d_qk"] == w["d_v"] and w["d_qk"] in (64, 128) and aligned:
        return "decode_ring_kernel"
    return "decode_kernel"


def source_digest(paths):
    """sha256 over the code of the given sources with comments and blank
    space removed (an edit to a comment leaves a kernel's record valid)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in paths:
        text = open(os.path.join(ROOT, f), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def committed_profile(workload):
    """The committed rocprofv3 record of the decode kernel on this workload
    (HBM bytes per launch from FETCH_SIZE/WRITE_SIZE, average launch duration
    from --kernel-trace --stats), or None if there is none or the kernel
    sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"decode_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    return rec if source_digest(rec["sources"]) == rec["source_digest"] else None


def cpu_baseline(w, inp, dec, budget_s=15.0):
    """The oracle, untuned, on a bounded sample of the same workload: up to
    half the budget of prefill compressions, then decode steps over those
    rows for the rest of it."""
    import numpy as np

    import oracle
    from kv_cache_compression_obs_amd import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    cfg = oracle.Config(n_q_heads=w["n_q_heads"], n_kv_heads=w["n_kv_heads"], d_qk=w["d_qk"],
                        d_v=w["d_v"], L_sink=w["L_sink"], K=w["K"], L_recent=w["L_recent"],
                        W=w["W"], pool=w["pool"], v_aliases_k=w["v_aliases_k"],
                        scale=w.get("scale", 0.0), rope_theta=w["rope_theta"], rope_begin=w["rope_begin"],
                        rope_end=w["rope_end"], dtype=w["dtype"])
    elem = 2 if w["dtype"] == "bf16" else 4
    pre_b, dec_b = algorithmic_bytes(dict(w, B=1), elem)
    t0 = time.perf_counter()
    n_req = 0
    results = []
    n_avail = inp["k"].shape[0]
    while n_req < n_avail and (time.perf_counter() - t0) < budget_s / 2:
        q = synth.to_f64(inp["q_obs"][n_req])
        k = synth.to_f64(inp["k"][n_req])
        v = synth.to_f64(inp["v"][n_req]) if inp["v"] is not None else None
        results.append(oracle.prefill_compress_one(cfg, q, k, v))
        n_req += 1
    t_pre = time.perf_counter() - t0
    state = oracle.CacheState(cfg, n_req)
    for i, r in enumerate(results):
        state.admit(i, r)
    t1 = time.perf_counter()
    n_dec = 0
    while n_dec < dec["q"].shape[0] and (time.perf_counter() - t1) < budget_s - t_pre:
        sl = slice(0, n_req)
        oracle.decode_step(state, synth.to_f64(dec["q"][n_dec][sl]),
                           synth.to_f64(dec["k_new"][n_dec][sl]),
                           synth.to_f64(dec["v_new"][n_dec][sl]) if dec["v_new"] is not None
                           else None, np.full(n_req, w["L"] + n_dec))
        n_dec += 1
    t_dec = time.perf_counter() - t1
    sample_bytes = n_req * pre_b + n_dec * n_req * dec_b
    return dict({
        "value": sample_bytes / (t_pre + t_dec) / 1e9,
        "unit": "GB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"fp64 oracle: prefill compression of {n_req} of {w['B']} requests "
                   f"({t_pre:.2f} s), then {n_dec} decode steps over those {n_req} rows "
                   f"({t_dec:.2f} s); same algorithmic-byte accounting as value"),
        "prefill_compress_ms_per_request": 1e3 * t_pre / max(n_req, 1),
        "decode_ms_per_row_step": 1e3 * t_dec / max(n_dec * n_req, 1),
    }, **host_info())


def given_lse_prefill(ss, torch, w, cfg, inp, reps=5):
    """ss_prefill_compress_lse (one score pass) on the same batch.  The
    observation rows' log-sum-exp, which a prefill attention hands over, is
    prepared beforehand with torch (fp32) and is not timed."""
    import math
    q, k = inp["q_obs"], inp["k"]
    b, Hq, W, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    scale = w.get("scale", 0.0) or 1.0 / math.sqrt(d)
    vis = torch.arange(L, device="cuda")[None, :] <= (L - W + torch.arange(W, device="cuda"))[:, None]
    lse = torch.empty(b, Hq, W, dtype=torch.float32, device="cuda")
    for bi in range(b):
        for h in range(Hkv):
            kt = k[bi, h].float().t().contiguous()
            z = scale * (q[bi, h * G:(h + 1) * G].float().reshape(G * W, d) @ kt)
            z = z.view(G, W, L).masked_fill(~vis, -math.inf)
            lse[bi, h * G:(h + 1) * G] = torch.logsumexp(z, dim=2)
    cache = ss.Cache(cfg, b)
    ws = torch.empty(ss.ss_prefill_workspace_bytes(cfg, b, L), dtype=torch.uint8, device="cuda")
    ss.ss_prefill_compress(cfg, q, k, inp["v"], cache, ws=ws, lse=lse)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        ss.ss_prefill_compress(cfg, q, k, inp["v"], cache, ws=ws, lse=lse)
    ev[1].record()
    torch.cuda.synchronize()
    return {"prefill_compress_ms_per_layer": round(ev[0].elapsed_time(ev[1]) / reps, 4),
            "note": "ss_prefill_compress_lse: one score pass over the middle keys, the rows' "
                    "log-sum-exp given"}


def varlen_admission(ss, torch, synth, w, cfg, reps=5):
    """Continuous-batching admission of B prompts of log-uniform lengths in
    [1024, L] (seeded): one ss_prefill_compress_varlen call against one
    ss_prefill_compress call per request."""
    B = w["B"]
    lens = synth.request_lengths(dict(w, len_min=min(1024, w["L"]), len_max=w["L"]), 3, B)
    reqs = [synth.prefill_inputs(w, 300 + i, device="cuda", B=1, L=n) for i, n in enumerate(lens)]
    q_obs = torch.cat([r["q_obs"] for r in reqs]).contiguous()
    k = torch.cat([r["k"][0] for r in reqs], dim=1).contiguous()
    v = (torch.cat([r["v"][0] for r in reqs], dim=1).contiguous()
         if reqs[0]["v"] is not None else None)
    cu = torch.tensor([0] + [sum(lens[:i + 1]) for i in range(B)], dtype=torch.int32,
                      device="cuda")
    max_L = max(lens)
    cache = ss.Cache(cfg, B)
    ws = torch.empty(ss.ss_prefill_workspace_bytes(cfg, B, max_L), dtype=torch.uint8,
                     device="cuda")
    rows = [torch.tensor([i], dtype=torch.int32, device="cuda") for i in range(B)]

    def one_call():
        ss.ss_prefill_compress_varlen(cfg, q_obs, k, v, cu, max_L, cache, ws=ws)

    def per_request():
        for i, r in enumerate(reqs):
            ss.ss_prefill_compress(cfg, r["q_obs"], r["k"], r["v"], cache, rows=rows[i], ws=ws)

    out = {}
    for name, fn in (("one_call_ms", one_call), ("per_request_calls_ms", per_request)):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        out[name] = round(ev[0].elapsed_time(ev[1]) / reps, 4)
    out.update(requests=B, compressed=sum(n > w["C"] for n in lens),
               length_range=[min(lens), max(lens)],
               speedup=round(out["per_request_calls_ms"] / out["one_call_ms"], 3))
    return out


def continuous_batching(ss, torch, synth, seed=5):
    """The continuous-batching workload as specified: 64 rows of 32q/8kv,
    d 128, bf16, C = 32768; requests of seeded log-uniform lengths in
    [1k, 128k], each set up through ss_prefill_compress (rows at or below
    capacity stored as they are); then 1000 decode steps, and before steps
    200, 400, 600 and 800 a seeded row's request finishes and a new
    65536-token prompt is compressed into that row (one single-row
    ss_prefill_compress).  The timed region is the 1000 steps with the four
    admissions; every input is resident beforehand."""
    w = synth.workload("llama8b_cb64")
    cfg = ss.make_config(**w)
    B, C, Hkv, d, steps = w["B"], w["C"], w["n_kv_heads"], w["d_qk"], w["steps"]
    lens = synth.request_lengths(w, seed, B)
    adm_rows = synth.admission_rows(w, seed)
    cache = ss.Cache(cfg, B)
    ws_p = torch.empty(ss.ss_prefill_workspace_bytes(cfg, 1, max(max(lens), w["L"])),
                       dtype=torch.uint8, device="cuda")
    for r, n in enumerate(lens):
        inp = synth.prefill_inputs(w, seed * 1000 + r, device="cuda", B=1, L=n)
        ss.ss_prefill_compress(cfg, inp["q_obs"], inp["k"], inp["v"], cache,
                               rows=torch.tensor([r], dtype=torch.int32, device="cuda"), ws=ws_p)
        del inp
    adm = {t: (r, synth.prefill_inputs(w, seed * 1000 + 500 + t, device="cuda", B=1, L=w["L"]),
               torch.tensor([r], dtype=torch.int32, device="cuda"))
           for t, r in zip(w["admissions"], adm_rows)}
    dec = synth.decode_inputs(w, seed, steps, device="cuda")
    # positions of every step, known in advance from the schedule
    n_tok = list(lens)
    pos_host, valid = [], 0
    for t in range(steps):
        if t in adm:
            n_tok[adm[t][0]] = w["L"]
        pos_host.append(list(n_tok))
        valid += sum(min(n + 1, C) for n in n_tok)
        n_tok = [n + 1 for n in n_tok]
    posbuf = torch.tensor(pos_host, dtype=torch.int32, device="cuda")
    out = torch.empty(B, w["n_q_heads"], d, dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = ss.decode_workspace(cfg, B)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 + 2 * len(adm))]
    torch.cuda.synchronize()
    ev[0].record()
    k = 0
    for t in range(steps):
        if t in adm:
            row, inp, rows = adm[t]
            ev[2 + 2 * k].record()
            ss.ss_prefill_compress(cfg, inp["q_obs"], inp["k"], inp["v"], cache, rows=rows,
                                   ws=ws_p)
            ev[3 + 2 * k].record()
            k += 1
        ss.ss_decode_step(cfg, dec["q"][t], dec["k_new"][t], dec["v_new"][t], posbuf[t], cache,
                          out, err, ws)
    ev[1].record()
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError("continuous batching: pos != n_tokens")
    total_s = ev[0].elapsed_time(ev[1]) / 1e3
    adm_s = sum(ev[2 + 2 * i].elapsed_time(ev[3 + 2 * i]) for i in range(len(adm))) / 1e3
    dec_s = total_s - adm_s
    bytes_dec = valid * Hkv * 2 * d * 2
    return {"rows": B, "cache_slots": C, "decode_steps": steps,
            "admissions": {str(t): {"row": r, "prompt": w["L"]} for t, (r, _, _) in adm.items()},
            "length_range": [min(lens), max(lens)],
            "rows_at_capacity": sum(n >= C for n in lens),
            "valid_slot_fraction": round(valid / (steps * B * C), 4),
            "total_ms": round(1e3 * total_s, 3),
            "admission_ms_each": round(1e3 * adm_s / max(len(adm), 1), 4),
            "decode_step_us": round(1e6 * dec_s / steps, 2),
            "decode_attn_GBps": round(bytes_dec / dec_s / 1e9, 1),
            "tokens_per_s_incl_admissions": round(B * steps / total_s, 1),
            "note": "GB/s over the valid slots only (per-request valid counts); tokens/s = "
                    "rows x steps over the whole timed region, admissions included"}


def uncompressed_baseline(ss, torch, hip, w, cfg, inp, dec, n_dec, R):
    """The same decode over a cache that keeps the whole prompt (C = L: the
    recent window widened to L - L_sink - K, so the prompt is stored as it is
    and every slot is valid), timed like the compressed decode: what the
    fixed-size cache saves per decode step (the caller divides by the
    compressed decode's launch time)."""
    B, L = w["B"], w["L"]
    wu = dict(w, L_recent=L - w["L_sink"] - w["K"])
    wu["C"] = L
    cfg_u = ss.make_config(**wu)
    caches = [ss.Cache(cfg_u, B) for _ in range(R)]
    for c in caches:
        ss.ss_prefill_compress(cfg_u, inp["q_obs"], inp["k"], inp["v"], c)
    ws = ss.decode_workspace(cfg_u, B)
    dt = ss.TORCH_DTYPE[cfg.dtype]
    out = torch.empty(B, w["n_q_heads"], w["d_v"], dtype=dt, device="cuda")
    n = min(n_dec, 64)
    pos = (L + torch.arange(n, dtype=torch.int32, device="cuda") // R)[:, None].repeat(1, B)
    ev = hip.create(2)
    for t in range(n):                     # warm-up pass at positions L.., then the timed pass
        vn = dec["v_new"][t] if dec["v_new"] is not None else None
        ss.ss_decode_step(cfg_u, dec["q"][t], dec["k_new"][t], vn, pos[t], caches[t % R], out,
                          ws=ws)
    pos += (n + R - 1) // R
    for t in range(n):
        vn = dec["v_new"][t] if dec["v_new"] is not None else None
        evs = (ev[0] if t == 0 else None, ev[1] if t == n - 1 else None)
        ss.ss_decode_step(cfg_u, dec["q"][t], dec["k_new"][t], vn, pos[t], caches[t % R], out,
                          ws=ws, events=evs if any(evs) else None)
    torch.cuda.synchronize()
    step_s = hip.elapsed_ms(ev[0], ev[1]) / n / 1e3
    hip.destroy(ev)
    elem = 2 if w["dtype"] == "bf16" else 4
    _, dec_b = algorithmic_bytes(wu, elem)
    return {
        "cache_slots": L,
        "decode_step_us": round(1e6 * step_s, 2),
        "decode_attn_GBps": round(dec_b / step_s / 1e9, 1),
        "kv_bytes_ratio": round(L / w["C"], 3),
        "note": f"{n} decode launches over a cache holding all {L} prompt tokens",
    }


def run_steps(ss, torch, synth, hip, w, steps, warmup, n_dec, R, inp=None, dec=None):
    """Build R compressed copies of the workload's cache, then run `warmup`
    untimed and `steps` timed steps (one ss_prefill_compress of the batch +
    n_dec ss_decode_step over the copies in turn).  The timed region is
    bracketed by device synchronisations; per-phase times come from events
    on the launch stream."""
    cfg = ss.make_config(**w)
    B, Hq, L = w["B"], w["n_q_heads"], w["L"]
    dt = synth.TORCH_DTYPE[w["dtype"]]
    if inp is None:
        inp = synth.prefill_inputs(w, seed=2, device="cuda")
    if dec is None:
        dec = synth.decode_inputs(w, seed=2, steps=n_dec, device="cuda")
    caches = [ss.Cache(cfg, B) for _ in range(R)]
    ws_p = torch.empty(ss.ss_prefill_workspace_bytes(cfg, B, L), dtype=torch.uint8, device="cuda")
    ws_d = ss.decode_workspace(cfg, B)
    out = torch.empty(B, Hq, w["d_v"], dtype=dt, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    total_steps = warmup + steps
    max_pos = total_steps * n_dec + 1
    posbuf = (L + torch.arange(max_pos, dtype=torch.int32, device="cuda"))[:, None].repeat(1, B)
    for c in caches:                       # every copy starts as a compressed prompt
        ss.ss_prefill_compress(cfg, inp["q_obs"], inp["k"], inp["v"], c, ws=ws_p)
    count = [0] * R
    ev_score = [hip.create(2) for _ in range(total_steps)]
    ev_attn = [hip.create(2) for _ in range(total_steps)]
    tev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(total_steps)]

    def step(i):
        e = tev[i]
        e[0].record()
        ss.ss_prefill_compress(cfg, inp["q_obs"], inp["k"], inp["v"], caches[0], ws=ws_p,
                               events=(ev_score[i][0], ev_score[i][1]))
        count[0] = 0
        e[1].record()
        ea = ev_attn[i]
        for t in range(n_dec):
            r = t % R
            vn = dec["v_new"][t] if dec["v_new"] is not None else None
            # one event right before the first decode kernel and one right
            # after the last: markers between launches would perturb them
            evs = (ea[0] if t == 0 else None, ea[1] if t == n_dec - 1 else None)
            ss.ss_decode_step(cfg, dec["q"][t], dec["k_new"][t], vn, posbuf[count[r]], caches[r],
                              out, err, ws_d, events=evs if any(evs) else None)
            count[r] += 1
        e[2].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup, total_steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if int(err.item()) != 0:
        raise RuntimeError("decode reported pos != n_tokens: the benchmark's bookkeeping is wrong")

    timed = range(warmup, total_steps)
    pre_ms = [tev[i][0].elapsed_time(tev[i][1]) for i in timed]
    dec_ms = [tev[i][1].elapsed_time(tev[i][2]) for i in timed]
    score_ms = [hip.elapsed_ms(ev_score[i][0], ev_score[i][1]) for i in timed]
    attn_ms = [hip.elapsed_ms(ev_attn[i][0], ev_attn[i][1]) / n_dec for i in timed]
    hip.destroy([e for p in ev_score for e in p] + [e for p in ev_attn for e in p])
    elem = 2 if w["dtype"] == "bf16" else 4
    pre_b, dec_b = algorithmic_bytes(w, elem)
    attn_avg_s = sum(attn_ms) / len(attn_ms) / 1e3
    dec_call_s = sum(dec_ms) / len(dec_ms) / 1e3 / n_dec
    fl_alg, fl_exec = score_flops(w)
    score_s = sum(score_ms) / len(score_ms) / 1e3
    achieved = dec_b / attn_avg_s / 1e9
    roof = {
        "kernel": decode_kernel_name(w) + " (RoPE + ring scatter + split-C flash-decode + merge)",
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": None,
        "avg_launch_us": round(1e6 * attn_avg_s, 3),
        "bytes_per_launch": dec_b,
        "timing": "HIP events on the launch stream: one right before the first decode "
                  "launch of a step, one right after its last; average = their distance / "
                  "launches (includes the gaps between back-to-back launches)",
    }
    prof = committed_profile(w["name"])
    if prof is not None:
        roof["traffic"] = prof["traffic_bytes"]
        if "rocprof_avg_us" in prof:
            roof["rocprof_avg_us"] = prof["rocprof_avg_us"]
            roof["frac_rocprof"] = round(dec_b / (prof["rocprof_avg_us"] * 1e-6) / 1e9
                                         / HBM_PEAK_GBPS, 4)
    kb = score_key_bytes(w, elem)
    return {
        "wall_s": wall, "step_bytes": pre_b + n_dec * dec_b, "inp": inp, "dec": dec,
        "decode_tokens_per_s_per_layer": round(B * n_dec * steps / wall, 1),
        "decode_tokens_per_s_model": round(B / (w["layers"] * dec_call_s), 1),
        "decode_attn_GBps": round(dec_b / dec_call_s / 1e9, 1),
        "decode_step_us": round(1e6 * dec_call_s, 2),
        "prefill_compress_ms_per_layer": round(sum(pre_ms) / len(pre_ms), 4),
        "attn_avg_s": attn_avg_s,
        "roofline": roof,
        "score_kernels": {
            "avg_us": round(1e6 * score_s, 2),
            "key_bytes": kb,
            "hbm_GBps": round(kb / score_s / 1e9, 1),
            "frac_hbm_peak": round(kb / score_s / 1e9 / HBM_PEAK_GBPS, 4),
            "tflops_algorithmic": round(fl_alg / score_s / 1e12, 2),
            "tflops_executed": round(fl_exec / score_s / 1e12, 2),
            "frac_bf16_peak_executed": round(fl_exec / score_s / 1e12 / BF16_PEAK_TFLOPS, 4),
        },
    }


def describe(w, n_dec, R):
    return (f"{w['name']}: batch {w['B']}, {w['n_q_heads']}q/{w['n_kv_heads']}kv heads, "
            f"d {w['d_qk']}{'' if not w['v_aliases_k'] else ' latent (value = first %d)' % w['d_v']}"
            f", prompt {w['L']} -> C={w['C']} ({w['L_sink']}+{w['K']}+{w['L_recent']}), "
            f"W={w['W']}, pool {w['pool']}, {n_dec} decode steps, {R} cache copies, "
            f"{w['layers']} layers in the model")


PUBLIC_KEYS = ("decode_tokens_per_s_per_layer", "decode_tokens_per_s_model", "decode_attn_GBps",
               "decode_step_us", "prefill_compress_ms_per_layer", "roofline", "score_kernels")


def run_leg(leg, ss, torch, synth, hip, R, n_dec=None):
    """One extra measurement, alone in its process: another workload's steps
    (2 timed, 8 warm-up) and its one-pass prefill (given log-sum-exp), the
    continuous-batching run, or the uncompressed baseline of a workload
    ("uncompressed:<workload>")."""
    if leg == "continuous_batching":
        return continuous_batching(ss, torch, synth)
    if leg.startswith("uncompressed:"):
        w = synth.workload(leg.split(":", 1)[1])
        n = n_dec or w["steps"]
        inp = synth.prefill_inputs(w, seed=2, device="cuda")
        dec = synth.decode_inputs(w, seed=2, steps=n, device="cuda")
        return uncompressed_baseline(ss, torch, hip, w, ss.make_config(**w), inp, dec, n, R)
    wo = synth.workload(leg)
    # 8 warm-up steps: in a fresh process the host needs about that long
    # before it issues decode launches faster than llama8b_c4k's 47 us
    # kernels complete (after 1 warm-up step the launches came 110-120 us
    # apart)
    inp = synth.prefill_inputs(wo, seed=2, device="cuda")
    ro = run_steps(ss, torch, synth, hip, wo, 2, 8, wo["steps"], R, inp=inp)
    res = dict({"config": describe(wo, wo["steps"], R)}, **{k: ro[k] for k in PUBLIC_KEYS})
    del ro
    torch.cuda.empty_cache()
    res["given_lse"] = given_lse_prefill(ss, torch, wo, ss.make_config(**wo), inp)
    return res


def leg_in_child(leg, R, n_dec):
    """run_leg in a fresh child process (this process waits for it).  In one
    process, decode over buffers allocated after another workload's were
    freed ran about 5% slower than in a fresh process (llama8b_128k 158.9
    against 166.1-166.4 us per launch, the latent layer 188 against 196 us):
    each measurement gets the memory state of a process that allocates its
    caches once, as a server does and as the profile runs do."""
    cmd = [sys.executable, os.path.abspath(__file__), "--leg", leg, "--replicas", str(R),
           "--decode-steps", str(n_dec)]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
    lines = p.stdout.strip().splitlines()
    if p.returncode != 0 or not lines:
        # reported in the line, which the headline measurement still carries
        print(f"bench.py: leg {leg} failed with status {p.returncode}", file=sys.stderr)
        return {"error": f"the leg's process ended with status {p.returncode}"}
    return json.loads(lines[-1])


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="deepseek_mla_128k")
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-uncompressed", action="store_true",
                    help="skip the uncompressed-cache baseline (decode over C = L slots)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the step only: skip the given-lse prefill, the varlen admission, "
                         "the other workloads, the continuous-batching run and the "
                         "uncompressed baseline (for profiling runs)")
    ap.add_argument("--leg", default=None,
                    help="run one extra measurement alone and print it as JSON: a workload "
                         "name, continuous_batching or uncompressed:<workload> (the full "
                         "bench runs each extra measurement this way, in a child process)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain elementwise copy of this many MiB first (a kernel of "
                         "known traffic, to calibrate FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; this library runs on one GPU "
              "(the multi-GPU sharding is a design note, not a code path)", file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cache_compression_obs_amd import snapstream as ss
    from kv_cache_compression_obs_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)       # reads and writes exactly n*4 bytes
        torch.cuda.synchronize()
        del src, dst
    R = max(1, args.replicas)
    hip = HipEvents()
    if args.leg is not None:
        print(json.dumps(run_leg(args.leg, ss, torch, synth, hip, R, args.decode_steps)),
              flush=True)
        return
    w = synth.workload(args.workload)
    cfg = ss.make_config(**w)
    n_dec = args.decode_steps or w["steps"]
    r = run_steps(ss, torch, synth, hip, w, args.steps, args.warmup, n_dec, R)
    inp, dec = r["inp"], r["dec"]
    res = {
        "metric": METRIC,
        "value": round(r["step_bytes"] * args.steps / r["wall_s"] / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * r["wall_s"] / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic",
        "config": {"workload": describe(w, n_dec, R),
                   "global_batch": w["B"], "seq_len": w["L"], "cache_slots": w["C"],
                   "decode_steps_per_step": n_dec, "layers_in_model": w["layers"],
                   "parallelism": "single GPU (one tensor-parallel rank's heads)"},
        "value_definition": "algorithmic HBM bytes of the step (prefill: prompt keys read once + "
                            "C cache rows gathered, read and written; decode: every valid cache "
                            "row read) per second of wall time",
    }
    for k in PUBLIC_KEYS:
        res[k] = r[k]
    if not args.no_extras:
        res["given_lse"] = given_lse_prefill(ss, torch, w, cfg, inp)
        res["varlen_admission"] = varlen_admission(ss, torch, synth, w, cfg)
    if not args.no_cpu_baseline:
        cpu_inp = {k: (v[:16] if v is not None else None) for k, v in inp.items()}
        cpu_dec = {k: (v.cpu() if v is not None else None) for k, v in dec.items()}
    attn_s = r["attn_avg_s"]
    del r, inp, dec
    torch.cuda.empty_cache()
    # each further measurement in a fresh child process (see leg_in_child)
    if not (args.no_uncompressed or args.no_extras):
        u = leg_in_child(f"uncompressed:{w['name']}", R, n_dec)
        if "decode_step_us" in u:
            u["decode_speedup_of_fixed_cache"] = round(u["decode_step_us"] / (1e6 * attn_s), 3)
        res["uncompressed_baseline"] = u
    if not args.no_extras:
        res["other_workloads"] = {
            name: leg_in_child(name, R, synth.workload(name)["steps"])
            for name in ("llama8b_c4k", "llama8b_128k", "deepseek_mla_128k") if name != w["name"]}
        res["continuous_batching"] = leg_in_child("continuous_batching", R, n_dec)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, cpu_inp, cpu_dec)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

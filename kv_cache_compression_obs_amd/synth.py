"""Seeded synthetic inputs for the SnapStream hot path.

This module only describes workloads (shapes and hyperparameters) and draws
random tensors for them.  It holds none of the method's arithmetic: no
scoring, pooling, selection, rotary embedding, slot arithmetic or attention.
Tests feed the same tensors to the library and to the CPU oracle; the
benchmark uses it to fill device memory.

Workloads (shapes of the layers the pages deploy: Llama-3.1-8B attention with
GQA and DeepSeek-R1 MLA at 128k context with a 32k fixed cache, the companion
page's configured L_recent = 31,744):

  tiny_fp32           1 x (4q/2kv) x d64, fp32, prompt 512 -> C=196 (4+64+128),
                      W=16, pool 7, 8 planted heavy keys per kv-head, 64 steps
  llama8b_c4k         16 x (32q/8kv) x d128, bf16, prompt 16384 -> C=4096
                      (64+1984+2048), W=32, pool 7, rope 5e5, 256 steps
  llama8b_128k        8 x (32q/8kv) x d128, bf16, prompt 131072 -> C=32768
                      (64+960+31744), W=32, pool 7, 32 layers, 512 steps
  deepseek_mla_128k   32 x (8q/1 latent) x d576 (value = first 512), bf16,
                      prompt 131072 -> C=32768, W=32, pool 7, rope 1e4 on
                      dims 512..575, softmax scale 1/sqrt(192) (the model's
                      per-head 128 + 64 query dims before absorption),
                      61 layers, 512 steps
  llama8b_cb64        64 rows x (32q/8kv) x d128, bf16, C=32768, request
                      lengths log-uniform in [1k, 128k], 1000 steps; before
                      steps 200/400/600/800 a seeded row's request is replaced
                      by a new 65536-token prompt
"""
from __future__ import annotations

import copy
import math

import numpy as np
import torch

# 1/sqrt(128 + 64) held exactly as the fp32 value the library receives
MLA_SCALE = float(np.float32(1.0 / math.sqrt(192.0)))

WORKLOADS = {
    "tiny_fp32": dict(
        B=1, n_q_heads=4, n_kv_heads=2, d_qk=64, d_v=64, v_aliases_k=False,
        L=512, L_sink=4, K=64, L_recent=128, W=16, pool=7, dtype="f32",
        rope_theta=0.0, rope_begin=0, rope_end=0, steps=64, layers=1,
        heavy_keys=8, heavy_scale=8.0, key_lognormal=False),
    "llama8b_c4k": dict(
        B=16, n_q_heads=32, n_kv_heads=8, d_qk=128, d_v=128, v_aliases_k=False,
        L=16384, L_sink=64, K=1984, L_recent=2048, W=32, pool=7, dtype="bf16",
        rope_theta=500000.0, rope_begin=0, rope_end=128, steps=256, layers=1,
        heavy_keys=0, heavy_scale=1.0, key_lognormal=True),
    "llama8b_128k": dict(
        B=8, n_q_heads=32, n_kv_heads=8, d_qk=128, d_v=128, v_aliases_k=False,
        L=131072, L_sink=64, K=960, L_recent=31744, W=32, pool=7, dtype="bf16",
        rope_theta=500000.0, rope_begin=0, rope_end=128, steps=512, layers=32,
        heavy_keys=0, heavy_scale=1.0, key_lognormal=True),
    "deepseek_mla_128k": dict(
        B=32, n_q_heads=8, n_kv_heads=1, d_qk=576, d_v=512, v_aliases_k=True,
        scale=MLA_SCALE, L=131072, L_sink=64, K=960, L_recent=31744, W=32, pool=7, dtype="bf16",
        rope_theta=10000.0, rope_begin=512, rope_end=576, steps=512, layers=61,
        heavy_keys=0, heavy_scale=1.0, key_lognormal=False),
    "llama8b_cb64": dict(
        B=64, n_q_heads=32, n_kv_heads=8, d_qk=128, d_v=128, v_aliases_k=False,
        L=65536, L_sink=64, K=960, L_recent=31744, W=32, pool=7, dtype="bf16",
        rope_theta=500000.0, rope_begin=0, rope_end=128, steps=1000, layers=1,
        heavy_keys=0, heavy_scale=1.0, key_lognormal=True,
        len_min=1024, len_max=131072, admissions=(200, 400, 600, 800)),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def workload(name: str, **overrides) -> dict:
    w = copy.deepcopy(WORKLOADS[name])
    w.update(overrides)
    w["name"] = name
    w["C"] = w["L_sink"] + w["K"] + w["L_recent"]
    return w


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(g, shape, device):
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)


def heavy_key_positions(w: dict, g: torch.Generator, device) -> torch.Tensor:
    """Positions of the planted heavy keys of one kv-head: inside the middle
    region [L_sink, L - L_recent), at least 3 from its edges, at least 8
    apart (one per equal-width bin, 4 clear of the bin edges)."""
    lo = w["L_sink"] + 3
    hi = w["L"] - w["L_recent"] - 4          # inclusive
    n = w["heavy_keys"]
    width = (hi - lo + 1) / n
    offs = torch.rand(n, generator=g, device=device)
    pos = []
    for j in range(n):
        b0 = lo + math.ceil(j * width) + 4
        b1 = lo + math.floor((j + 1) * width) - 4
        pos.append(b0 + int(offs[j].item() * (b1 - b0 + 1)) if b1 >= b0 else b0)
    return torch.tensor(pos, dtype=torch.long)


def prefill_inputs(w: dict, seed: int, device="cpu", B: int | None = None,
                   L: int | None = None) -> dict:
    """q_obs [B, Hq, W, d_qk], k [B, Hkv, L, d_qk], v [B, Hkv, L, d_v] (None
    when the value aliases the latent key), in the workload's dtype.  Values
    stand for post-rotary queries and keys: i.i.d. N(0, 1) is invariant in
    distribution under rotation.  Draw order: q_obs, k, v, key-norm factors,
    heavy keys."""
    B = w["B"] if B is None else B
    L = w["L"] if L is None else L
    Hq, Hkv, dq, dv = w["n_q_heads"], w["n_kv_heads"], w["d_qk"], w["d_v"]
    g = _gen(seed, device)
    dt = TORCH_DTYPE[w["dtype"]]
    q_obs = _randn(g, (B, Hq, w["W"], dq), device).to(dt)
    k = _randn(g, (B, Hkv, L, dq), device)
    v = None if w["v_aliases_k"] else _randn(g, (B, Hkv, L, dv), device).to(dt)
    if w["key_lognormal"]:
        k *= torch.exp(0.5 * _randn(g, (B, Hkv, L, 1), device))
    if w["heavy_keys"] and L > w["C"]:      # planted only where the prompt gets compressed
        ww = dict(w, L=L)
        for b in range(B):
            for h in range(Hkv):
                pos = heavy_key_positions(ww, g, device)
                k[b, h, pos.to(device)] *= w["heavy_scale"]
    return dict(q_obs=q_obs, k=k.to(dt), v=v)


def decode_inputs(w: dict, seed: int, steps: int, device="cpu", B: int | None = None) -> dict:
    """Per-step pre-rotary q [steps, B, Hq, d_qk], k_new [steps, B, Hkv, d_qk],
    v_new [steps, B, Hkv, d_v] (None when aliased).  Draw order: q, k_new,
    v_new, key-norm factors."""
    B = w["B"] if B is None else B
    Hq, Hkv, dq, dv = w["n_q_heads"], w["n_kv_heads"], w["d_qk"], w["d_v"]
    g = _gen(seed + 1_000_003, device)
    dt = TORCH_DTYPE[w["dtype"]]
    q = _randn(g, (steps, B, Hq, dq), device).to(dt)
    k_new = _randn(g, (steps, B, Hkv, dq), device)
    v_new = None if w["v_aliases_k"] else _randn(g, (steps, B, Hkv, dv), device).to(dt)
    if w["key_lognormal"]:
        k_new *= torch.exp(0.5 * _randn(g, (steps, B, Hkv, 1), device))
    return dict(q=q, k_new=k_new.to(dt), v_new=v_new)


def request_lengths(w: dict, seed: int, n: int) -> list[int]:
    """Continuous-batching request lengths, log-uniform in [len_min, len_max]."""
    g = _gen(seed + 7_777, "cpu")
    u = torch.rand(n, generator=g, dtype=torch.float64)
    lo, hi = math.log(w["len_min"]), math.log(w["len_max"])
    return [int(round(math.exp(lo + float(x) * (hi - lo)))) for x in u]


def admission_rows(w: dict, seed: int) -> list[int]:
    """Continuous-batching schedule: the distinct rows (seeded) whose requests
    finish and are replaced by a new prompt, one per step of w["admissions"]."""
    g = _gen(seed + 9_999, "cpu")
    return torch.randperm(w["B"], generator=g)[:len(w["admissions"])].tolist()


def to_f64(t):
    """Exact float64 copy of a tensor's stored values (for the oracle)."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()

"""Plain, slow, fp64 CPU oracle for the SnapStream hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product (the HIP library and its
Python binding) never imports, calls or falls back to it, and it shares no
code, table or helper with that path.

Sources (the pages this follows):
  [ABS]  "SnapStream: Efficient Long Sequence Decoding on Dataflow Accelerators",
         abstract (fixed-size cache from StreamingLLM + SnapKV; static graphs and
         continuous batching; Llama-3.1-8B and DeepSeek-R1 models).
  [COMP] "SnapStream: Taming KV-Cache Eviction for Dataflow Accelerators"
         (episode companion page), sections "Two Ingredients, Fused",
         "Fixed-Size Cache Layout", "Ring Buffer vs. Naive Slicing",
         "Why This Wasn't Already Standard", "Prefill / Decode Pipeline",
         "Infinity-Bench KV Retrieval: The Failure Mode" (pooling-based top-K).
  [MAP]  the citation-map page for arXiv 2511.03092, "Builds on" list
         (SnapKV, StreamingLLM attention sinks, GQA, DeepSeek-V2 MLA).

The pages give no formulas.  Where they are silent this file takes the
plainest reading the rest supports; each such reading is marked READING and
is listed in the design notes of the repository.

Every floating-point quantity is float64.  Inputs arrive as float64 arrays that
hold the exact values of the I/O dtype (fp32 or bf16); nothing is re-rounded
except where the method itself stores a freshly computed value into the cache
(the rotated decode key), which is rounded once, to nearest-even, to the cache
dtype.

Parity pins: every function here is pinned by CPU tests against closed forms,
invariants, brute force on tiny inputs, or library routines (torch SDPA,
scipy softmax, Python's stable sort).  The cache-layout conventions (ring
phase, ascending order of the top-K segment, rotate-half RoPE) are choices the
pages cannot fix; they are pinned against their own closed forms only.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


# --------------------------------------------------------------------------
# configuration (the oracle's own copy; the library has its own C struct)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Config:
    """Hyperparameters of one attention layer and its fixed cache.

    [COMP] "Fixed-Size Cache Layout": the segment sizes L_sink, K and L_recent
    are configurable hyperparameters.  W (observation window) and pool (pool
    width) are the SnapKV knobs named in [COMP] "Two Ingredients, Fused" and
    "Infinity-Bench KV Retrieval" (pooling-based top-K).
    """
    n_q_heads: int
    n_kv_heads: int
    d_qk: int
    d_v: int
    L_sink: int
    K: int
    L_recent: int
    W: int
    pool: int
    v_aliases_k: bool = False      # MLA: the value is the first d_v dims of the latent
    scale: float = 0.0             # 0 -> 1/sqrt(d_qk)
    rope_theta: float = 0.0        # 0 -> no rotary embedding at decode
    rope_begin: int = 0
    rope_end: int = 0              # rotate dims [rope_begin, rope_end)
    dtype: str = "f32"             # storage dtype of the cache: "f32" or "bf16"

    @property
    def C(self) -> int:
        return self.L_sink + self.K + self.L_recent

    @property
    def G(self) -> int:
        assert self.n_q_heads % self.n_kv_heads == 0
        return self.n_q_heads // self.n_kv_heads

    @property
    def sm_scale(self) -> float:
        return self.scale if self.scale != 0.0 else 1.0 / math.sqrt(self.d_qk)


# --------------------------------------------------------------------------
# rounding to the storage dtype
# --------------------------------------------------------------------------
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even, in one
    step (no intermediate fp32 rounding).  bf16 keeps 8 significant bits and
    fp32's exponent range; values below 2**-126 sit on the fixed subnormal grid
    of spacing 2**-133."""
    x = np.asarray(x, dtype=np.float64)
    mant, exp = np.frexp(x)                      # x = mant * 2**exp, 0.5 <= |mant| < 1
    normal = np.rint(mant * 256.0) * np.ldexp(1.0, exp - 8)
    sub = np.rint(x * 2.0 ** 133) * 2.0 ** -133
    out = np.where(np.abs(x) >= 2.0 ** -126, normal, sub)
    return np.where(x == 0, x, out)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# rotary position embedding (decode side)
# --------------------------------------------------------------------------
def rope_inv_freq(theta: float, d_rot: int) -> np.ndarray:
    """inv_freq_i = theta ** (-2 i / d_rot), i = 0 .. d_rot/2 - 1.
    READING: the standard rotate-half rotary embedding, with no frequency
    rescaling; the pages say nothing about positional encoding."""
    i = np.arange(d_rot // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / d_rot)


def rope_rotate(x: np.ndarray, pos: int, theta: float, begin: int, end: int) -> np.ndarray:
    """Rotate the last axis of x (float64) at absolute position pos over dims
    [begin, end): pairs (begin + i, begin + i + h), h = (end - begin) / 2.

    READING: keys are stored already rotated at their original absolute
    positions, so attention over the cache does not depend on the slot a key
    occupies ([COMP] "Ring Buffer vs. Naive Slicing" rotates only slot indices,
    never positions)."""
    y = np.array(x, dtype=np.float64, copy=True)
    if theta == 0.0 or end <= begin:
        return y
    h = (end - begin) // 2
    ang = float(pos) * rope_inv_freq(theta, end - begin)
    c, s = np.cos(ang), np.sin(ang)
    x1 = y[..., begin:begin + h].copy()
    x2 = y[..., begin + h:end].copy()
    y[..., begin:begin + h] = x1 * c - x2 * s
    y[..., begin + h:end] = x2 * c + x1 * s
    return y


# --------------------------------------------------------------------------
# prefill: observation-window scores, pooling, top-K, cache layout
# --------------------------------------------------------------------------
def obs_column_scores(q_obs: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Column scores of one (request, kv-head) group over ALL prompt keys.

    q_obs: [G, W, d] the observation-window queries of the G q-heads that share
           this kv-head (post-RoPE), i.e. the queries at prompt positions
           L-W .. L-1.
    k:     [L, d] the group's prompt keys (post-RoPE).
    Returns col [L] with col[i] = sum_g sum_r softmax_r(scale * q_{g,r} . k)[i].

    SnapKV scoring ([MAP] SnapKV; [COMP] "Two Ingredients, Fused": attention-
    based token selection).  READING: each observation query takes the causal
    softmax of the model's own attention over the whole prompt up to its own
    position (key i is visible to row r iff i <= L - W + r); probabilities are
    summed (not averaged) over the window and over the q-heads of the GQA group.
    """
    G, W, d = q_obs.shape
    L = k.shape[0]
    col = np.zeros(L, dtype=np.float64)
    row_pos = L - W + np.arange(W)
    visible = np.arange(L)[None, :] <= row_pos[:, None]          # [W, L]
    for g in range(G):
        z = scale * (q_obs[g] @ k.T)                              # [W, L]
        z = np.where(visible, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        e = np.exp(z)
        p = e / e.sum(axis=1, keepdims=True)
        col += p.sum(axis=0)
    return col


def max_pool_clipped(raw: np.ndarray, P: int) -> np.ndarray:
    """pooled[i] = max{ raw[u] : 0 <= u < m, |u - i| <= (P-1)/2 }.

    [COMP] "Infinity-Bench KV Retrieval" names pooling-based top-K selection.
    READING: max-pool of odd width P, stride 1, same length as the input, the
    window clipped to the middle region (equivalent to -inf padding), so sink
    and recent scores never enter."""
    assert P >= 1 and P % 2 == 1
    m = raw.shape[0]
    p = (P - 1) // 2
    padded = np.concatenate([np.full(p, -np.inf), raw, np.full(p, -np.inf)])
    win = np.lib.stride_tricks.sliding_window_view(padded, P)     # [m, P]
    return win.max(axis=1)


def select_topk(pooled: np.ndarray, K: int) -> np.ndarray:
    """The K best middle positions in the total order (pooled descending,
    index ascending), returned in ascending index order.

    READING: ties go to the lower index; the kept tokens are stored in
    ascending position order (attention does not depend on this order, the
    slot map does)."""
    m = pooled.shape[0]
    assert 0 <= K <= m
    order = np.lexsort((np.arange(m), -pooled))
    return np.sort(order[:K])


def ring_slot(t: int, S: int, K: int, R: int) -> int:
    """Slot of absolute position t.  Positions below S+K keep slot t (sinks,
    and the first tokens of an uncompressed prompt); from S+K on, positions
    cycle through the recent window [S+K, S+K+R).

    [COMP] "Ring Buffer vs. Naive Slicing": decode only rotates the recent
    window, writing into a fixed index.  READING: the ring phase is measured
    from the ring start S+K, which makes an uncompressed prompt lay out as
    slot = t, keeps the valid slots a prefix, and makes every write evict
    exactly position t - R."""
    if t < S + K:
        return t
    return S + K + ((t - S - K) % R)


@dataclasses.dataclass
class PrefillResult:
    col: np.ndarray | None       # [Hkv, L] column scores (None if not compressed)
    raw: np.ndarray | None       # [Hkv, m]
    pooled: np.ndarray | None    # [Hkv, m]
    sel: np.ndarray | None       # [Hkv, K] ascending indices into the middle region
    k_cache: np.ndarray          # [Hkv, C, d_qk]
    v_cache: np.ndarray | None   # [Hkv, C, d_v] (None when v aliases k)
    slot_pos: np.ndarray         # [Hkv, C] int64, -1 = empty
    n_tokens: int


def prefill_compress_one(cfg: Config, q_obs: np.ndarray, k: np.ndarray,
                         v: np.ndarray | None) -> PrefillResult:
    """Build the fixed-size cache of one request.

    q_obs [Hq, W, d_qk], k [Hkv, L, d_qk], v [Hkv, L, d_v] (or None if v aliases
    k), all post-RoPE, float64 holding I/O-dtype values.

    [COMP] "Fixed-Size Cache Layout": built once at prefill as sink tokens +
    SnapKV top-K middle + recent window.  [ABS]: StreamingLLM sinks/recency
    fused with SnapKV selection.  When L <= C nothing is scored and token t
    goes to slot t (READING)."""
    S, K, R, C = cfg.L_sink, cfg.K, cfg.L_recent, cfg.C
    Hkv, L, _ = k.shape
    G = cfg.G

    if L <= C:
        k_cache = np.zeros((Hkv, C, cfg.d_qk))
        v_cache = None if cfg.v_aliases_k else np.zeros((Hkv, C, cfg.d_v))
        slot_pos = np.full((Hkv, C), -1, dtype=np.int64)
        for h in range(Hkv):
            k_cache[h, :L] = k[h]
            if v_cache is not None:
                v_cache[h, :L] = v[h]
            slot_pos[h, :L] = np.arange(L)
        return PrefillResult(None, None, None, None, k_cache, v_cache, slot_pos, L)

    assert cfg.W <= R, "the observation window must lie inside the recent window"
    m = L - R - S
    cols = np.zeros((Hkv, L))
    raws = np.zeros((Hkv, m))
    pools = np.zeros((Hkv, m))
    sels = np.zeros((Hkv, K), dtype=np.int64)
    for h in range(Hkv):
        col = obs_column_scores(q_obs[h * G:(h + 1) * G], k[h], cfg.sm_scale)
        raw = col[S:L - R]
        pooled = max_pool_clipped(raw, cfg.pool)
        sel = select_topk(pooled, K)
        cols[h], raws[h], pools[h], sels[h] = col, raw, pooled, sel
    k_cache, v_cache, slot_pos = fixed_cache_layout(cfg, k, v, sels)
    return PrefillResult(cols, raws, pools, sels, k_cache, v_cache, slot_pos, L)


def fixed_cache_layout(cfg: Config, k: np.ndarray, v: np.ndarray | None, sel: np.ndarray):
    """The fixed cache of one compressed request (L > C) from its kept middle
    tokens sel [Hkv, K] (ascending indices into the middle region): returns
    (k_cache [Hkv, C, d_qk], v_cache [Hkv, C, d_v] or None, slot_pos [Hkv, C]).

    [COMP] "Fixed-Size Cache Layout": sink tokens, then the selected middle
    tokens, then the recent window.  READING: sinks and selected tokens take
    slots 0 .. S+K-1 in position order; recent token t goes to its ring slot
    ([COMP] "Ring Buffer vs. Naive Slicing")."""
    S, K, R, C = cfg.L_sink, cfg.K, cfg.L_recent, cfg.C
    Hkv, L, _ = k.shape
    k_cache = np.zeros((Hkv, C, cfg.d_qk))
    v_cache = None if cfg.v_aliases_k else np.zeros((Hkv, C, cfg.d_v))
    slot_pos = np.full((Hkv, C), -1, dtype=np.int64)
    for h in range(Hkv):
        tokens = list(range(S)) + [S + int(j) for j in sel[h]] + list(range(L - R, L))
        for t_idx, t in enumerate(tokens):
            slot = t_idx if t_idx < S + K else ring_slot(t, S, K, R)
            k_cache[h, slot] = k[h, t]
            if v_cache is not None:
                v_cache[h, slot] = v[h, t]
            slot_pos[h, slot] = t
    return k_cache, v_cache, slot_pos


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------
class CacheState:
    """The fixed-shape cache of B_max request rows (float64 arrays that hold
    I/O-dtype values).  Shapes never change after construction ([COMP]
    "Why This Wasn't Already Standard": static shapes)."""

    def __init__(self, cfg: Config, B_max: int):
        self.cfg = cfg
        C = cfg.C
        self.k = np.zeros((B_max, cfg.n_kv_heads, C, cfg.d_qk))
        self.v = None if cfg.v_aliases_k else np.zeros((B_max, cfg.n_kv_heads, C, cfg.d_v))
        self.slot_pos = np.full((B_max, cfg.n_kv_heads, C), -1, dtype=np.int64)
        self.n_tokens = np.zeros(B_max, dtype=np.int64)

    def admit(self, row: int, res: PrefillResult) -> None:
        """Place one request's prefill result into a batch row (continuous
        batching, [ABS] and [COMP] "Why This Wasn't Already Standard")."""
        self.k[row] = res.k_cache
        if self.v is not None:
            self.v[row] = res.v_cache
        self.slot_pos[row] = res.slot_pos
        self.n_tokens[row] = res.n_tokens

    def values(self, row: int) -> np.ndarray:
        if self.v is not None:
            return self.v[row]
        return self.k[row][..., :self.cfg.d_v]


def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q . keys^T) . vals for one query vector q [d]."""
    z = scale * (keys @ q)
    z = z - z.max()
    e = np.exp(z)
    return (e / e.sum()) @ vals


def decode_write(state: CacheState, k_new: np.ndarray, v_new: np.ndarray | None,
                 pos: np.ndarray) -> bool:
    """The cache update of one decode step for every row (no attention).

    k_new [B, Hkv, d_qk] (pre-RoPE), v_new [B, Hkv, d_v] or None when v
    aliases k, pos [B] absolute positions (< 0: inactive row).

    [COMP] "Ring Buffer vs. Naive Slicing": the new key/value is scattered into
    a fixed slot of the recent window (no gather, no concatenation), evicting
    position pos - L_recent.  READING: RoPE at the absolute position, the
    rotated key rounded once to the cache dtype.  Returns True if some active
    row had pos != n_tokens (the write is applied at pos anyway)."""
    cfg = state.cfg
    err = False
    for b in range(k_new.shape[0]):
        p = int(pos[b])
        if p < 0:
            continue
        if p != state.n_tokens[b]:
            err = True
        slot = ring_slot(p, cfg.L_sink, cfg.K, cfg.L_recent)
        kr = rope_rotate(k_new[b], p, cfg.rope_theta, cfg.rope_begin, cfg.rope_end)
        state.k[b, :, slot] = round_to_dtype(kr, cfg.dtype)
        if state.v is not None:
            state.v[b, :, slot] = v_new[b]
        state.slot_pos[b, :, slot] = p
        state.n_tokens[b] = p + 1
    return err


def decode_step(state: CacheState, q: np.ndarray, k_new: np.ndarray,
                v_new: np.ndarray | None, pos: np.ndarray):
    """One decode step for every row.

    q [B, Hq, d_qk], k_new [B, Hkv, d_qk] (pre-RoPE), v_new [B, Hkv, d_v] or
    None when v aliases k, pos [B] absolute positions (< 0: inactive row).

    The cache update is decode_write; attention then runs over every valid
    slot of the fixed cache ([COMP] "Prefill / Decode Pipeline": decode is a
    memory-bound pass over the cache).  READING: the new token is written
    before attention and attends to itself; the valid slots of a row are its
    first min(n_tokens, C) slots.  Returns (out [B, Hq, d_v], err) where err is
    True if some active row had pos != n_tokens (the step is applied at pos
    anyway)."""
    cfg = state.cfg
    B = q.shape[0]
    G, C = cfg.G, cfg.C
    out = np.zeros((B, cfg.n_q_heads, cfg.d_v))
    err = decode_write(state, k_new, v_new, pos)
    for b in range(B):
        p = int(pos[b])
        if p < 0:
            continue
        n_valid = min(p + 1, C)
        vals = state.values(b)
        for j in range(cfg.n_q_heads):
            h = j // G
            qr = rope_rotate(q[b, j], p, cfg.rope_theta, cfg.rope_begin, cfg.rope_end)
            out[b, j] = attend(qr, state.k[b, h, :n_valid], vals[h, :n_valid], cfg.sm_scale)
    return out, err

"""ctypes binding of libsnapstream's C ABI (include/snapstream.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels of libsnapstream.so.  PyTorch supplies device memory and the stream.
Raises if the shared library has not been built (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsnapstream.so")

(SS_OK, SS_ERR_INVALID_ARG, SS_ERR_UNSUPPORTED, SS_ERR_WORKSPACE, SS_ERR_HIP,
 SS_ERR_SCRATCH_LIMIT) = range(6)
SS_F32, SS_BF16 = 0, 1
DTYPES = {"f32": SS_F32, "bf16": SS_BF16}
TORCH_DTYPE = {SS_F32: torch.float32, SS_BF16: torch.bfloat16}

EXPORTS = ("ss_cache_slots", "ss_prefill_workspace_bytes", "ss_decode_workspace_bytes",
           "ss_decode_workspace_init", "ss_prefill_compress", "ss_decode_step",
           "ss_prefill_compress_timed", "ss_decode_step_timed", "ss_prefill_compress_lse",
           "ss_prefill_compress_lse_timed", "ss_prefill_compress_varlen",
           "ss_prefill_compress_varlen_timed", "ss_decode_step_noalloc", "ss_status_string")


class ss_config(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("v_aliases_k", ctypes.c_int32),
        ("L_sink", ctypes.c_int32), ("K", ctypes.c_int32), ("L_recent", ctypes.c_int32),
        ("W", ctypes.c_int32), ("pool", ctypes.c_int32),
        ("scale", ctypes.c_float), ("rope_theta", ctypes.c_float),
        ("rope_begin", ctypes.c_int32), ("rope_end", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class ss_cache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("slot_pos", ctypes.c_void_p), ("n_tokens", ctypes.c_void_p),
        ("B_max", ctypes.c_int32),
    ]


class SnapStreamError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libsnapstream.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m kv_cache_compression_obs_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
        L.ss_cache_slots.argtypes = [P(ss_config)]
        L.ss_cache_slots.restype = I32
        L.ss_prefill_workspace_bytes.argtypes = [P(ss_config), I32, I32]
        L.ss_prefill_workspace_bytes.restype = SZ
        L.ss_decode_workspace_bytes.argtypes = [P(ss_config), I32]
        L.ss_decode_workspace_bytes.restype = SZ
        L.ss_prefill_compress.argtypes = [P(ss_config), VP, VP, VP, I32, I32, VP, P(ss_cache),
                                          VP, VP, VP, VP, SZ, VP]
        L.ss_prefill_compress.restype = I32
        L.ss_decode_step.argtypes = [P(ss_config), VP, VP, VP, VP, P(ss_cache), VP, VP, VP, SZ, VP]
        L.ss_decode_step.restype = I32
        L.ss_prefill_compress_timed.argtypes = L.ss_prefill_compress.argtypes + [VP, VP]
        L.ss_prefill_compress_timed.restype = I32
        L.ss_decode_step_timed.argtypes = L.ss_decode_step.argtypes + [VP, VP]
        L.ss_decode_step_timed.restype = I32
        L.ss_prefill_compress_lse.argtypes = [P(ss_config), VP, VP, VP, I32, I32, VP, VP,
                                              P(ss_cache), VP, VP, VP, VP, SZ, VP]
        L.ss_prefill_compress_lse.restype = I32
        L.ss_prefill_compress_lse_timed.argtypes = L.ss_prefill_compress_lse.argtypes + [VP, VP]
        L.ss_prefill_compress_lse_timed.restype = I32
        L.ss_prefill_compress_varlen.argtypes = [P(ss_config), VP, VP, VP, I32, VP, I32, VP, VP,
                                                 P(ss_cache), VP, VP, VP, VP, SZ, VP]
        L.ss_prefill_compress_varlen.restype = I32
        L.ss_prefill_compress_varlen_timed.argtypes = (L.ss_prefill_compress_varlen.argtypes +
                                                       [VP, VP])
        L.ss_prefill_compress_varlen_timed.restype = I32
        L.ss_decode_step_noalloc.argtypes = [P(ss_config), VP, VP, VP, VP, P(ss_cache), VP, VP,
                                             VP]
        L.ss_decode_step_noalloc.restype = I32
        L.ss_decode_workspace_init.argtypes = [P(ss_config), I32, VP, SZ, VP]
        L.ss_decode_workspace_init.restype = I32
        L.ss_status_string.argtypes = [I32]
        L.ss_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ss_status_string(int(status)).decode()


def make_config(n_q_heads, n_kv_heads, d_qk, d_v, L_sink, K, L_recent, W, pool,
                v_aliases_k=False, scale=0.0, rope_theta=0.0, rope_begin=0, rope_end=0,
                dtype="bf16", **_ignored) -> ss_config:
    return ss_config(int(n_q_heads), int(n_kv_heads), int(d_qk), int(d_v), int(bool(v_aliases_k)),
                     int(L_sink), int(K), int(L_recent), int(W), int(pool), float(scale),
                     float(rope_theta), int(rope_begin), int(rope_end),
                     DTYPES[dtype] if isinstance(dtype, str) else int(dtype))


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream, t) -> int:
    """The raw handle of `stream`, by default the current stream of the
    device that holds tensor t (the device the call's buffers live on)."""
    if stream is None:
        stream = torch.cuda.current_stream(t.get_device())
    return stream.cuda_stream


def _check(t, name, dtype=None, shape=None):
    """A contiguous device tensor of the given dtype and, where given, shape:
    the kernels index every tensor by the shape the config implies, so a
    smaller tensor would be read or written out of bounds on the device."""
    if t is None:
        return
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_cache(cfg: ss_config, cache: "Cache"):
    C = ss_cache_slots(cfg)
    dt = TORCH_DTYPE[cfg.dtype]
    B, H = cache.B_max, cfg.n_kv_heads
    _check(cache.k, "cache.k", dt, (B, H, C, cfg.d_qk))
    if cfg.v_aliases_k:
        if cache.v is not None:
            raise ValueError("cache.v must be None when the value aliases the key")
    else:
        _check(cache.v, "cache.v", dt, (B, H, C, cfg.d_v))
        if cache.v is None:
            raise ValueError("cache.v is required")
    _check(cache.slot_pos, "cache.slot_pos", torch.int32, (B, H, C))
    _check(cache.n_tokens, "cache.n_tokens", torch.int32, (B,))


def ss_cache_slots(cfg: ss_config) -> int:
    return lib().ss_cache_slots(ctypes.byref(cfg))


def ss_prefill_workspace_bytes(cfg: ss_config, b: int, L: int) -> int:
    return lib().ss_prefill_workspace_bytes(ctypes.byref(cfg), int(b), int(L))


def ss_decode_workspace_bytes(cfg: ss_config, B_max: int) -> int:
    return lib().ss_decode_workspace_bytes(ctypes.byref(cfg), int(B_max))


def ss_decode_workspace_init(cfg: ss_config, B_max: int, ws, stream=None) -> None:
    _check(ws, "ws", torch.uint8)
    st = lib().ss_decode_workspace_init(ctypes.byref(cfg), int(B_max), _ptr(ws), ws.numel(),
                                        _stream(stream, ws))
    if st != SS_OK:
        raise SnapStreamError(st, "ss_decode_workspace_init")


def decode_workspace(cfg: ss_config, B_max: int, device="cuda"):
    """A decode workspace ready for its first ss_decode_step (zero-filled)."""
    return torch.zeros(ss_decode_workspace_bytes(cfg, B_max), dtype=torch.uint8, device=device)


class Cache:
    """Device tensors of the fixed-shape cache (caller-owned, never resized)."""

    def __init__(self, cfg: ss_config, B_max: int, device="cuda"):
        C = ss_cache_slots(cfg)
        if C < 0:
            raise ValueError("invalid config")
        dt = TORCH_DTYPE[cfg.dtype]
        self.cfg, self.B_max, self.C = cfg, B_max, C
        self.k = torch.zeros(B_max, cfg.n_kv_heads, C, cfg.d_qk, dtype=dt, device=device)
        self.v = None if cfg.v_aliases_k else torch.zeros(B_max, cfg.n_kv_heads, C, cfg.d_v,
                                                          dtype=dt, device=device)
        self.slot_pos = torch.full((B_max, cfg.n_kv_heads, C), -1, dtype=torch.int32,
                                   device=device)
        self.n_tokens = torch.zeros(B_max, dtype=torch.int32, device=device)

    def struct(self) -> ss_cache:
        return ss_cache(_ptr(self.k), _ptr(self.v), _ptr(self.slot_pos), _ptr(self.n_tokens),
                        self.B_max)

    def clone(self) -> "Cache":
        c = Cache.__new__(Cache)
        c.cfg, c.B_max, c.C = self.cfg, self.B_max, self.C
        c.k = self.k.clone()
        c.v = None if self.v is None else self.v.clone()
        c.slot_pos, c.n_tokens = self.slot_pos.clone(), self.n_tokens.clone()
        return c


def ss_prefill_compress(cfg: ss_config, q_obs, k, v, cache: Cache, rows=None, raw_out=None,
                        pooled_out=None, sel_out=None, ws=None, stream=None,
                        events=None, lse=None) -> None:
    """Build the fixed cache of b = k.shape[0] requests of L = k.shape[2] tokens
    into `cache` (rows `rows`, default 0..b-1).  events: optional pair of raw
    hipEvent_t handles recorded around the score kernels.  lse: optional
    float32 [b, n_q_heads, W] log-sum-exp of the observation rows; given, the
    call goes to ss_prefill_compress_lse (one score pass)."""
    dt = TORCH_DTYPE[cfg.dtype]
    if k is None or k.dim() != 4:
        raise ValueError("k must be [b, n_kv_heads, L, d_qk]")
    b, L = int(k.shape[0]), int(k.shape[2])
    H, Hq, C = cfg.n_kv_heads, cfg.n_q_heads, ss_cache_slots(cfg)
    m = max(L - cfg.L_sink - cfg.L_recent, 0)
    _check(k, "k", dt, (b, H, L, cfg.d_qk))
    if cfg.v_aliases_k:
        if v is not None:
            raise ValueError("v must be None when the value aliases the key")
    else:
        if v is None:
            raise ValueError("v is required")
        _check(v, "v", dt, (b, H, L, cfg.d_v))
    if L > C or q_obs is not None:
        if q_obs is None:
            raise ValueError("q_obs is required when the prompt is compressed")
        _check(q_obs, "q_obs", dt, (b, Hq, cfg.W, cfg.d_qk))
    _check(rows, "rows", torch.int32, (b,))
    if rows is None and b > cache.B_max:
        raise ValueError(f"{b} requests do not fit a cache of {cache.B_max} rows")
    for t, n in ((raw_out, "raw_out"), (pooled_out, "pooled_out")):
        _check(t, n, torch.float32, (b, H, m))
    _check(sel_out, "sel_out", torch.int32, (b, H, cfg.K))
    _check_cache(cfg, cache)
    if ws is None:
        ws = torch.empty(ss_prefill_workspace_bytes(cfg, b, L), dtype=torch.uint8,
                         device=k.device)
    cs = cache.struct()
    tail = (_ptr(rows), ctypes.byref(cs), _ptr(raw_out), _ptr(pooled_out), _ptr(sel_out),
            _ptr(ws), ws.numel(), _stream(stream, k))
    head = (ctypes.byref(cfg), _ptr(q_obs), _ptr(k), _ptr(v), b, L)
    if lse is not None:
        _check(lse, "lse", torch.float32, (b, Hq, cfg.W))
        args, name = head + (_ptr(lse),) + tail, "ss_prefill_compress_lse"
    else:
        args, name = head + tail, "ss_prefill_compress"
    if events is None:
        st = getattr(lib(), name)(*args)
    else:
        st = getattr(lib(), name + "_timed")(*args, events[0], events[1])
    if st != SS_OK:
        raise SnapStreamError(st, name)


def ss_prefill_compress_varlen(cfg: ss_config, q_obs, k, v, cu_seqlens, max_L: int,
                               cache: Cache, rows=None, lse=None, raw_out=None, pooled_out=None,
                               sel_out=None, ws=None, stream=None, events=None) -> None:
    """Build the fixed cache of b = q_obs.shape[0] requests of different
    lengths: k [n_kv_heads, T, d_qk] and v packed per kv-head, request i =
    tokens cu_seqlens[i] .. cu_seqlens[i+1]-1 (int32 device [b+1]); max_L bounds
    every length.  lse: optional [b, n_q_heads, W] (one-pass scoring)."""
    dt = TORCH_DTYPE[cfg.dtype]
    if q_obs is None or q_obs.dim() != 4 or k is None or k.dim() != 3:
        raise ValueError("q_obs must be [b, n_q_heads, W, d_qk] and k [n_kv_heads, T, d_qk]")
    b, T = int(q_obs.shape[0]), int(k.shape[1])
    H, Hq = cfg.n_kv_heads, cfg.n_q_heads
    m = max(int(max_L) - cfg.L_sink - cfg.L_recent, 0)
    _check(q_obs, "q_obs", dt, (b, Hq, cfg.W, cfg.d_qk))
    _check(k, "k", dt, (H, T, cfg.d_qk))
    if cfg.v_aliases_k:
        if v is not None:
            raise ValueError("v must be None when the value aliases the key")
    else:
        if v is None:
            raise ValueError("v is required")
        _check(v, "v", dt, (H, T, cfg.d_v))
    _check(cu_seqlens, "cu_seqlens", torch.int32, (b + 1,))
    _check(rows, "rows", torch.int32, (b,))
    if rows is None and b > cache.B_max:
        raise ValueError(f"{b} requests do not fit a cache of {cache.B_max} rows")
    _check(lse, "lse", torch.float32, (b, Hq, cfg.W))
    for t, n in ((raw_out, "raw_out"), (pooled_out, "pooled_out")):
        _check(t, n, torch.float32, (b, H, m))
    _check(sel_out, "sel_out", torch.int32, (b, H, cfg.K))
    _check_cache(cfg, cache)
    if ws is None:
        ws = torch.empty(ss_prefill_workspace_bytes(cfg, b, max_L), dtype=torch.uint8,
                         device=k.device)
    cs = cache.struct()
    args = (ctypes.byref(cfg), _ptr(q_obs), _ptr(k), _ptr(v), b, _ptr(cu_seqlens), int(max_L),
            _ptr(lse), _ptr(rows), ctypes.byref(cs), _ptr(raw_out), _ptr(pooled_out),
            _ptr(sel_out), _ptr(ws), ws.numel(), _stream(stream, k))
    if events is None:
        st = lib().ss_prefill_compress_varlen(*args)
    else:
        st = lib().ss_prefill_compress_varlen_timed(*args, events[0], events[1])
    if st != SS_OK:
        raise SnapStreamError(st, "ss_prefill_compress_varlen")


def _check_decode(cfg, q, k_new, v_new, pos, cache, out, err_flag):
    dt = TORCH_DTYPE[cfg.dtype]
    B, H, Hq = cache.B_max, cfg.n_kv_heads, cfg.n_q_heads
    for t, n in ((q, "q"), (k_new, "k_new"), (out, "out"), (pos, "pos")):
        if t is None:
            raise ValueError(f"{n} is required")
    _check(q, "q", dt, (B, Hq, cfg.d_qk))
    _check(k_new, "k_new", dt, (B, H, cfg.d_qk))
    if cfg.v_aliases_k:
        if v_new is not None:
            raise ValueError("v_new must be None when the value aliases the key")
    else:
        if v_new is None:
            raise ValueError("v_new is required")
        _check(v_new, "v_new", dt, (B, H, cfg.d_v))
    _check(out, "out", dt, (B, Hq, cfg.d_v))
    _check(pos, "pos", torch.int32, (B,))
    _check(err_flag, "err_flag", torch.int32)
    if err_flag is not None and err_flag.numel() < 1:
        raise ValueError("err_flag must hold at least one int32")
    _check_cache(cfg, cache)


def ss_decode_step(cfg: ss_config, q, k_new, v_new, pos, cache: Cache, out, err_flag=None,
                   ws=None, stream=None, events=None) -> None:
    """One decode step of every cache row; writes `out` [B_max, Hq, d_v].
    events: optional pair of raw hipEvent_t handles recorded around the
    attention kernel."""
    _check_decode(cfg, q, k_new, v_new, pos, cache, out, err_flag)
    if ws is None:
        ws = decode_workspace(cfg, cache.B_max, q.device)
    cs = cache.struct()
    args = (ctypes.byref(cfg), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(pos), ctypes.byref(cs),
            _ptr(out), _ptr(err_flag), _ptr(ws), ws.numel(), _stream(stream, q))
    if events is None:
        st = lib().ss_decode_step(*args)
    else:
        st = lib().ss_decode_step_timed(*args, events[0], events[1])
    if st != SS_OK:
        raise SnapStreamError(st, "ss_decode_step")


def ss_decode_step_noalloc(cfg: ss_config, q, k_new, v_new, pos, cache: Cache, out,
                           err_flag=None, stream=None) -> None:
    """ss_decode_step without a workspace: the library's static device scratch
    holds the split partials (calls on one GPU must not overlap)."""
    _check_decode(cfg, q, k_new, v_new, pos, cache, out, err_flag)
    cs = cache.struct()
    st = lib().ss_decode_step_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(k_new), _ptr(v_new),
                                      _ptr(pos), ctypes.byref(cs), _ptr(out), _ptr(err_flag),
                                      _stream(stream, q))
    if st != SS_OK:
        raise SnapStreamError(st, "ss_decode_step_noalloc")

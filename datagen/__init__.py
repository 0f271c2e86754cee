"""Seeded synthetic inputs for the absorbed Gated-MLA layer.

This module is shared by the CPU oracle side and the HIP side of the tests and
the benchmark.  It only draws random numbers and rounds them to the storage
dtype; it contains none of the layer's arithmetic.

Recipe (shapes follow the MLA variable table of the "符号表" page and the
toy/full-size table of the "K3 混合架构" page):

* every tensor is drawn from its own counter-based Philox4x64 stream, keyed by
  ``(seed, tensor_id << 32 | chunk)``, so a tensor never depends on the size or
  order of the others; large tensors are drawn in independent chunks of
  ``max(1, 2**21 // cols)`` rows;
* ``q ~ N(0,1)`` with shape ``[B,T,H,d_q]`` (prefill) or ``[B,H,d_q]`` (decode);
* ``c`` is a row-wise RMS-normalised ``N(0,1)`` draw over the last axis
  (gain 1, ``eps = 1e-6`` inside the square root), computed in float64;
* ``W_UK [H,d_q,r]`` and ``W_UV [H,d_v,r]`` are ``N(0, 1/r)``;
* ``gate`` (pre-sigmoid logits) ``~ N(0,1)`` with shape ``[B,T,H*d_v]`` or
  ``[B,H*d_v]``;
* full-layer forward: ``x ~ N(0,1)`` ``[B,T,D]``; every projection weight
  (``W_kv_down [r,D]``, ``W_q_down [q_rank,D]``, ``W_q_up [H*d_q,q_rank]``,
  ``W_gate [H*d_v,D]``, ``W_o [D,H*d_v]``) is ``N(0, 1/in_features)``, so
  the gate logits and q come out near ``N(0,1)`` as above; the two norm
  gains are ``1 + N(0, 0.01)``;
* KDA (variable table of the "符号表" page: q, k ``[B,T,H,K]``, v
  ``[B,T,H_V,V]``, the log-space decay g ``[B,T,H_V,K]``, the write strength
  beta ``[B,T,H_V]``, the state ``[B,H_V,K,V]``): q and k rows are
  ``N(0,1)`` draws normalised to unit L2 norm (float64), q then times
  ``K**-0.5`` (the table's q already carries the scale); ``v ~ N(0,1)``;
  ``g = max(gate_low, -exp(N(-2, 1)))`` with ``gate_low = -5`` (the gate's
  lower bound on the same page), float32; ``beta = sigmoid(N(0,1))``,
  float32; an initial state, when asked for, ``N(0, 1/K)`` float32;
* decode cache lengths are i.i.d. uniform integers on ``[len_lo, len_hi]``;
  ``cu_seqlens`` is their int32 exclusive prefix sum;
* float64 draws are rounded to float32 (round-to-nearest-even) and, for bf16
  storage, float32 is rounded to bf16 (round-to-nearest-even).

Storage: bf16 tensors are returned as ``numpy.uint16`` bit patterns, float32
tensors as ``numpy.float32``.  ``as_f32`` returns the exact float32 value of
either, which is what the oracle consumes.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32 = "f32"
BF16 = "bf16"

_TID = {"q": 1, "c": 2, "w_uk": 3, "w_uv": 4, "gate": 5, "lens": 6, "x": 7, "w_kv_down": 8,
        "kv_norm": 9, "w_q_down": 10, "q_norm": 11, "w_q_up": 12, "w_gate": 13, "w_o": 14,
        "kda_q": 15, "kda_k": 16, "kda_v": 17, "kda_g": 18, "kda_beta": 19, "kda_s0": 20}
_CHUNK_ELEMS = 1 << 21
_RMS_EPS = 1e-6


def _gen(seed: int, tid: int, chunk: int) -> np.random.Generator:
    key = np.array([seed & 0xFFFFFFFFFFFFFFFF, (tid << 32) | chunk], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rnd = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rnd) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 value of bf16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f32(x: np.ndarray) -> np.ndarray:
    """Exact float32 view of a stored tensor (bf16 bits or float32)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    if dtype == F32:
        return x32
    raise ValueError(f"unknown dtype {dtype!r}")


def _draw_rows(seed: int, name: str, rows: int, cols: int, std: float, dtype: str,
               rms_norm: bool = False, mean: float = 0.0) -> np.ndarray:
    """rows x cols standard-normal draw (times std), chunked by rows."""
    out = np.empty((rows, cols), dtype=np.uint16 if dtype == BF16 else np.float32)
    chunk_rows = max(1, _CHUNK_ELEMS // cols)
    nchunks = max(1, -(-rows // chunk_rows))

    def work(ci: int) -> None:
        r0 = ci * chunk_rows
        r1 = min(rows, r0 + chunk_rows)
        if r1 <= r0:
            return
        x = _gen(seed, _TID[name], ci).standard_normal((r1 - r0, cols))
        if rms_norm:
            x = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + _RMS_EPS)
        elif std != 1.0:
            x = x * std
        if mean != 0.0:
            x = x + mean
        out[r0:r1] = _store(x, dtype)

    workers = min(nchunks, int(os.environ.get("DATAGEN_THREADS", "8")))
    if workers <= 1:
        for ci in range(nchunks):
            work(ci)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def prefill_inputs(B: int, T: int, H: int, d_q: int, d_v: int, r: int,
                   dtype: str = BF16, seed: int = 0) -> dict:
    """Inputs of one prefill call; all arrays row-major contiguous."""
    if min(B, T, H, d_q, d_v, r) <= 0:
        raise ValueError("all sizes must be positive")
    q = _draw_rows(seed, "q", B * T * H, d_q, 1.0, dtype).reshape(B, T, H, d_q)
    c = _draw_rows(seed, "c", B * T, r, 1.0, dtype, rms_norm=True).reshape(B, T, r)
    w_uk = _draw_rows(seed, "w_uk", H * d_q, r, r ** -0.5, dtype).reshape(H, d_q, r)
    w_uv = _draw_rows(seed, "w_uv", H * d_v, r, r ** -0.5, dtype).reshape(H, d_v, r)
    gate = _draw_rows(seed, "gate", B * T, H * d_v, 1.0, dtype).reshape(B, T, H * d_v)
    return dict(q=q, c=c, w_uk=w_uk, w_uv=w_uv, gate=gate,
                B=B, T=T, H=H, d_q=d_q, d_v=d_v, r=r, dtype=dtype, seed=seed)


def forward_inputs(B: int, T: int, D: int, q_rank: int, H: int, d_q: int, d_v: int, r: int,
                   dtype: str = BF16, seed: int = 0) -> dict:
    """Inputs of one full-layer forward: the activations x and every weight,
    laid out as linear layers (out_features x in_features)."""
    if min(B, T, D, q_rank, H, d_q, d_v, r) <= 0:
        raise ValueError("all sizes must be positive")
    x = _draw_rows(seed, "x", B * T, D, 1.0, dtype).reshape(B, T, D)
    w_kv_down = _draw_rows(seed, "w_kv_down", r, D, D ** -0.5, dtype)
    kv_norm = _draw_rows(seed, "kv_norm", 1, r, 0.1, dtype, mean=1.0).reshape(r)
    w_q_down = _draw_rows(seed, "w_q_down", q_rank, D, D ** -0.5, dtype)
    q_norm = _draw_rows(seed, "q_norm", 1, q_rank, 0.1, dtype, mean=1.0).reshape(q_rank)
    w_q_up = _draw_rows(seed, "w_q_up", H * d_q, q_rank, q_rank ** -0.5, dtype)
    w_uk = _draw_rows(seed, "w_uk", H * d_q, r, r ** -0.5, dtype).reshape(H, d_q, r)
    w_uv = _draw_rows(seed, "w_uv", H * d_v, r, r ** -0.5, dtype).reshape(H, d_v, r)
    w_gate = _draw_rows(seed, "w_gate", H * d_v, D, D ** -0.5, dtype)
    w_o = _draw_rows(seed, "w_o", D, H * d_v, (H * d_v) ** -0.5, dtype)
    return dict(x=x, w_kv_down=w_kv_down, kv_norm=kv_norm, w_q_down=w_q_down, q_norm=q_norm,
                w_q_up=w_q_up, w_uk=w_uk, w_uv=w_uv, w_gate=w_gate, w_o=w_o,
                B=B, T=T, D=D, q_rank=q_rank, H=H, d_q=d_q, d_v=d_v, r=r, dtype=dtype, seed=seed)


FORWARD_KEYS = ("x", "w_kv_down", "kv_norm", "w_q_down", "q_norm", "w_q_up", "w_uk", "w_uv", "w_gate", "w_o")


def _draw_f32(seed: int, name: str, shape, fn) -> np.ndarray:
    """float32 array of the given shape from fn(standard-normal float64 draw)."""
    n = int(np.prod(shape))
    x = _gen(seed, _TID[name], 0).standard_normal(n)
    return _store(fn(x), F32).reshape(shape)


def kda_inputs(B: int, T: int, H: int, G: int, K: int, V: int, dtype: str = BF16, seed: int = 0,
               gate_low: float = -5.0, init_state: bool = False) -> dict:
    """Inputs of one chunk_kda call: H query/key heads, H_V = G H value heads."""
    if min(B, T, H, G, K, V) <= 0:
        raise ValueError("all sizes must be positive")
    HV = G * H

    def unit_rows(name, rows, cols, mult):
        out = np.empty((rows, cols), dtype=np.uint16 if dtype == BF16 else np.float32)
        x = _gen(seed, _TID[name], 0).standard_normal((rows, cols))
        x = x / np.sqrt(np.sum(x * x, axis=1, keepdims=True)) * mult
        out[:] = _store(x, dtype)
        return out

    q = unit_rows("kda_q", B * T * H, K, K ** -0.5).reshape(B, T, H, K)
    k = unit_rows("kda_k", B * T * H, K, 1.0).reshape(B, T, H, K)
    v = _draw_rows(seed, "kda_v", B * T * HV, V, 1.0, dtype).reshape(B, T, HV, V)
    g = _draw_f32(seed, "kda_g", (B, T, HV, K), lambda x: np.maximum(gate_low, -np.exp(x - 2.0)))
    beta = _draw_f32(seed, "kda_beta", (B, T, HV), lambda x: 1.0 / (1.0 + np.exp(-x)))
    s0 = _draw_f32(seed, "kda_s0", (B, HV, K, V), lambda x: x * K ** -0.5) if init_state else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, s0=s0, B=B, T=T, H=H, G=G, K=K, V=V, dtype=dtype, seed=seed)


def decode_lengths(B: int, len_lo: int, len_hi: int, seed: int = 0) -> np.ndarray:
    """i.i.d. uniform integer cache lengths on [len_lo, len_hi] (inclusive)."""
    if not (1 <= len_lo <= len_hi):
        raise ValueError("need 1 <= len_lo <= len_hi")
    return _gen(seed, _TID["lens"], 0).integers(len_lo, len_hi + 1, size=B).astype(np.int64)


def decode_inputs(B: int, H: int, d_q: int, d_v: int, r: int, dtype: str = BF16,
                  seed: int = 0, len_lo: int = 1024, len_hi: int = 32768,
                  lengths=None) -> dict:
    """Inputs of one decode call against a packed latent cache."""
    lens = (np.asarray(lengths, dtype=np.int64) if lengths is not None
            else decode_lengths(B, len_lo, len_hi, seed))
    if lens.shape != (B,) or (lens < 1).any():
        raise ValueError("lengths must be B positive integers")
    cu = np.zeros(B + 1, dtype=np.int64)
    np.cumsum(lens, out=cu[1:])
    if cu[-1] >= 2 ** 31:
        raise ValueError("total cache length exceeds int32")
    total = int(cu[-1])
    q = _draw_rows(seed, "q", B * H, d_q, 1.0, dtype).reshape(B, H, d_q)
    c_cache = _draw_rows(seed, "c", total, r, 1.0, dtype, rms_norm=True)
    w_uk = _draw_rows(seed, "w_uk", H * d_q, r, r ** -0.5, dtype).reshape(H, d_q, r)
    w_uv = _draw_rows(seed, "w_uv", H * d_v, r, r ** -0.5, dtype).reshape(H, d_v, r)
    gate = _draw_rows(seed, "gate", B, H * d_v, 1.0, dtype).reshape(B, H * d_v)
    return dict(q=q, c_cache=c_cache, cu_seqlens=cu.astype(np.int32), lengths=lens,
                w_uk=w_uk, w_uv=w_uv, gate=gate,
                B=B, H=H, d_q=d_q, d_v=d_v, r=r, dtype=dtype, seed=seed,
                max_len=int(lens.max()))


def paged_layout(lengths, page_size: int, seed: int = 0, spare_pages: int = 3) -> dict:
    """A shuffled page assignment for sequences of the given lengths: sequence
    i gets ceil(len_i / page_size) pages drawn without replacement from a pool
    of (their total + spare_pages) pages.  block_table [B, max_pages] int32;
    entries past a sequence's pages are -1."""
    lens = np.asarray(lengths, dtype=np.int64)
    need = -(-lens // page_size)
    max_pages = int(need.max())
    num_pages = int(need.sum()) + spare_pages
    perm = _gen(seed, _TID["lens"], 1).permutation(num_pages)
    bt = np.full((len(lens), max_pages), -1, dtype=np.int32)
    o = 0
    for i, n in enumerate(need):
        bt[i, :n] = perm[o:o + n]
        o += n
    return dict(block_table=bt, num_pages=num_pages, max_pages=max_pages, page_size=page_size)


def scatter_to_pages(rows: np.ndarray, cu, layout: dict, fill=np.nan) -> np.ndarray:
    """Places packed rows [N, r] (storage dtype) of the sequences delimited by
    cu into a page pool [num_pages, page_size, r] following layout; slots no
    sequence owns hold `fill` (rounded to the storage dtype)."""
    ps, npg = layout["page_size"], layout["num_pages"]
    r = rows.shape[1]
    if rows.dtype == np.uint16:
        fb = f32_to_bf16_bits(np.array([fill], dtype=np.float32))[0]
        pool = np.full((npg, ps, r), fb, dtype=np.uint16)
    else:
        pool = np.full((npg, ps, r), fill, dtype=rows.dtype)
    bt = layout["block_table"]
    for i in range(len(cu) - 1):
        n = int(cu[i + 1] - cu[i])
        for p in range(-(-n // ps)):
            u0, u1 = p * ps, min(n, (p + 1) * ps)
            pool[bt[i, p], :u1 - u0] = rows[cu[i] + u0:cu[i] + u1]
    return pool


# Named workloads: the pages' toy and full-scale shapes.  Seeds are
# 0x4D4C41 + index so each workload draws independent data.
SEED_BASE = 0x4D4C41

WORKLOADS = {
    "toy_f32": dict(kind="prefill", B=2, T=128, H=8, d_q=16, d_v=16, r=32, dtype=F32,
                    scale=1.0, seed=SEED_BASE + 0),
    "toy_max": dict(kind="prefill", B=4, T=2048, H=8, d_q=16, d_v=16, r=32, dtype=BF16,
                    scale=16 ** -0.5, seed=SEED_BASE + 1),
    "mid": dict(kind="prefill", B=4, T=4096, H=32, d_q=64, d_v=64, r=256, dtype=BF16,
                scale=64 ** -0.5, seed=SEED_BASE + 2),
    "full_prefill": dict(kind="prefill", B=1, T=8192, H=96, d_q=128, d_v=128, r=512,
                         dtype=BF16, scale=128 ** -0.5, seed=SEED_BASE + 3),
    "full_decode": dict(kind="decode", B=64, H=96, d_q=128, d_v=128, r=512, dtype=BF16,
                        len_lo=1024, len_hi=32768, scale=128 ** -0.5, seed=SEED_BASE + 4),
    # the whole layer at the pages' toy and full widths (D, q_lora_rank from
    # the toy/full table of the "K3 混合架构" page)
    "toy_forward": dict(kind="forward", B=2, T=128, D=256, q_rank=64, H=8, d_q=16, d_v=16, r=32,
                        dtype=BF16, scale=16 ** -0.5, eps=1e-6, seed=SEED_BASE + 5),
    "full_forward": dict(kind="forward", B=1, T=8192, D=7168, q_rank=1536, H=96, d_q=128, d_v=128,
                         r=512, dtype=BF16, scale=128 ** -0.5, eps=1e-6, seed=SEED_BASE + 6),
    # chunk_kda at the pages' toy widths (H = H_V = 8, K = V = 16, T in the
    # 128-2048 range of the shape table) and the full K3 widths (H = H_V = 96,
    # K = V = 128) over the same 8192 positions as the MLA workloads
    "toy_kda": dict(kind="kda", B=2, T=512, H=8, G=1, K=16, V=16, dtype=BF16, seed=SEED_BASE + 7),
    "full_kda": dict(kind="kda", B=1, T=8192, H=96, G=1, K=128, V=128, dtype=BF16, seed=SEED_BASE + 8),
}


def workload_inputs(name: str) -> dict:
    w = dict(WORKLOADS[name])
    kind = w.pop("kind")
    if kind == "kda":
        d = kda_inputs(**w)
        d["kind"] = kind
        return d
    scale = w.pop("scale")
    eps = w.pop("eps", None)
    if kind == "prefill":
        d = prefill_inputs(**w)
    elif kind == "forward":
        d = forward_inputs(**w)
        d["eps"] = eps
    else:
        d = decode_inputs(**w)
    d["scale"] = scale
    d["kind"] = kind
    return d

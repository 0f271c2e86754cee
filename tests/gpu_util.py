"""Shared helpers for the GPU tests: seeded inputs to device tensors, calls
through the binding, and the parity bars.

Tolerances: bf16 storage with fp32 accumulation is compared element by
element with |gpu - oracle| <= 2e-2 (absolute); fp32 with
|gpu - oracle| <= 1e-4 * |oracle| + 1e-6.
"""
from __future__ import annotations

import numpy as np

import datagen as dg

BF16_ATOL = 2e-2
F32_RTOL, F32_ATOL = 1e-4, 1e-6


def torch():
    import torch as t
    return t


def to_dev(x: np.ndarray):
    t = torch()
    if x.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(t.bfloat16).cuda()
    if x.dtype == np.float32:
        return t.from_numpy(np.ascontiguousarray(x)).cuda()
    if x.dtype == np.int32:
        return t.from_numpy(np.ascontiguousarray(x)).cuda()
    raise TypeError(x.dtype)


def to_host_f64(t) -> np.ndarray:
    tt = torch()
    if t.dtype == tt.bfloat16:
        u = t.contiguous().view(tt.int16).cpu().numpy().view(np.uint16)
        return dg.bf16_bits_to_f32(u).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def run_prefill(d, scale=None):
    import rank_latent_causal_amd as mla
    args = [to_dev(d[k]) for k in ("q", "c", "w_uk", "w_uv", "gate")]
    out = mla.mla_absorb_prefill(*args, d["scale"] if scale is None else scale)
    torch().cuda.synchronize()
    return out


def run_extend(d, T, scale=None):
    """The last T positions of each sequence of prefill-shaped inputs d as a
    chunk over the whole latent (S = d's T rows)."""
    import rank_latent_causal_amd as mla
    S = d["T"]
    args = [to_dev(d["q"][:, S - T:]), to_dev(d["c"]), to_dev(d["w_uk"]), to_dev(d["w_uv"]),
            to_dev(d["gate"][:, S - T:])]
    out = mla.mla_absorb_extend(*args, d["scale"] if scale is None else scale)
    torch().cuda.synchronize()
    return out


def oracle_extend(o, d, T, rows=None, scale=None):
    f = dg.as_f32
    S = d["T"]
    return o.extend(f(d["q"])[:, S - T:], f(d["c"]), f(d["w_uk"]), f(d["w_uv"]), f(d["gate"])[:, S - T:],
                    d["scale"] if scale is None else scale, rows=rows)


def run_decode(d, scale=None, num_splits=0):
    import rank_latent_causal_amd as mla
    args = [to_dev(d["q"]), to_dev(d["c_cache"]), to_dev(d["cu_seqlens"]), to_dev(d["w_uk"]),
            to_dev(d["w_uv"]), to_dev(d["gate"])]
    out = mla.mla_absorb_decode(*args, d["scale"] if scale is None else scale, num_splits=num_splits)
    torch().cuda.synchronize()
    return out


def oracle_prefill(o, d, rows=None, scale=None):
    f = dg.as_f32
    return o.prefill(f(d["q"]), f(d["c"]), f(d["w_uk"]), f(d["w_uv"]), f(d["gate"]),
                     d["scale"] if scale is None else scale, rows=rows)


def oracle_decode(o, d, seqs=None, scale=None):
    f = dg.as_f32
    return o.decode(f(d["q"]), f(d["c_cache"]), d["cu_seqlens"].astype(np.int64), f(d["w_uk"]),
                    f(d["w_uv"]), f(d["gate"]), d["scale"] if scale is None else scale, seqs=seqs)


def assert_parity(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype == dg.BF16:
        bad = err > BF16_ATOL
        bar = f"atol {BF16_ATOL}"
    else:
        bad = err > F32_RTOL * np.abs(ref) + F32_ATOL
        bar = f"rtol {F32_RTOL} + atol {F32_ATOL}"
    if bad.any():
        idx = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {err.size} elements beyond {bar}; "
                             f"max err {err.max():.4g} at {idx} (gpu {got[idx]:.6g}, oracle {ref[idx]:.6g})")
    return float(err.max())


def sample_rows(B: int, T: int, n_random: int, seed: int) -> np.ndarray:
    """Flattened b*T+t rows: first/last positions, tile edges +-1 near both
    ends, and seeded random picks, in every batch."""
    rng = np.random.default_rng(seed)
    ts = {0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, T - 33, T - 32, T - 31, T - 17, T - 16, T - 2, T - 1}
    ts |= set(int(x) for x in rng.integers(0, T, size=n_random))
    ts = sorted(t for t in ts if 0 <= t < T)
    return np.array([b * T + t for b in range(B) for t in ts], dtype=np.int64)


def run_forward(d, eps=None, scale=None):
    """Full-layer forward of forward-shaped inputs d (bf16) through the binding."""
    import rank_latent_causal_amd as mla
    args = [to_dev(d[k]) for k in dg.FORWARD_KEYS]
    out = mla.mla_gated_forward(*args, d["eps"] if eps is None else eps, d["scale"] if scale is None else scale)
    torch().cuda.synchronize()
    return out


def oracle_forward(o, d, rows=None, eps=None, scale=None):
    """The oracle's full-layer forward with bf16 storage of the stage results."""
    return o.forward(*[dg.as_f32(d[k]) for k in dg.FORWARD_KEYS], d["eps"] if eps is None else eps,
                     d["scale"] if scale is None else scale, stage=o.STAGE_BF16, rows=rows)

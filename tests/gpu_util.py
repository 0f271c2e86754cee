"""Shared helpers for the GPU tests: seeded inputs to device tensors, calls
through the binding, and the parity bars.

Tolerances: bf16 storage with fp32 accumulation is compared element by
element with |gpu - oracle| <= 2e-2 (absolute); fp32 with
|gpu - oracle| <= 1e-4 * |oracle| + 1e-6.

At the full widths the outputs have an RMS near 0.025, about the size of
the absolute bar, so the element bar alone would pass a kernel that is a
few percent off everywhere.  Every comparison therefore also bounds
normwise relative errors ||gpu - oracle||_2 / ||oracle||_2:
  * of each output row (the last axis: one (b, t) position, or one decode
    sequence): 1e-2 (bf16), 1e-4 (fp32);
  * where the caller names the head width d_v, of each head over all rows:
    1e-2 (bf16), 1e-4 (fp32) -- a head scaled 2% off fails here;
  * and of each head block of each row (d_v elements): 2e-2 (bf16), 1e-4
    (fp32) -- a wrong head in a single row fails here.
The bf16 chain rounds q_abs, P and o_lat / l to bf16 (2^-9 relative each)
and the output itself.  Measured on the test workloads at the default
softmax scales: rows at most 0.006, head blocks of 128 elements at most
0.008; a 16-element head block (the toy widths) is a ratio of two short
sums and reached 0.016, and at four times the default scale (a peakier
softmax, see the accuracy regime of the bf16 path) rows reached 0.0084 and
blocks 0.017.  The achieved maximum absolute error and the maximum row,
head and block errors are printed (and appended as JSON lines to the file
named by MLA_PARITY_LOG, if set).
"""
from __future__ import annotations

import numpy as np

import datagen as dg

BF16_ATOL = 2e-2
F32_RTOL, F32_ATOL = 1e-4, 1e-6
BF16_NORM_REL = 1e-2   # per row and per head (all rows), normwise
BF16_BLOCK_REL = 2e-2  # per head block of one row, normwise
F32_NORM_REL = 1e-4


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


def _normwise(got: np.ndarray, ref: np.ndarray, width: int) -> np.ndarray:
    """||gpu - oracle|| / ||oracle|| over consecutive groups of `width`
    elements of the last axis (a group whose oracle norm is zero is measured
    against 1, i.e. absolutely)."""
    g = got.reshape(-1, width)
    r = ref.reshape(-1, width)
    den = np.linalg.norm(r, axis=1)
    return np.linalg.norm(g - r, axis=1) / np.where(den > 0, den, 1.0)


def assert_parity(got: np.ndarray, ref: np.ndarray, dtype: str, what: str, block: int | None = None):
    """Element bar plus the normwise bars per row (last axis) and, with
    `block` (the head width d_v), per head over all rows and per head block
    of each row."""
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype == dg.BF16:
        bad = err > BF16_ATOL
        bar = f"atol {BF16_ATOL}"
        nbar, bbar = BF16_NORM_REL, BF16_BLOCK_REL
    else:
        bad = err > F32_RTOL * np.abs(ref) + F32_ATOL
        bar = f"rtol {F32_RTOL} + atol {F32_ATOL}"
        nbar = bbar = F32_NORM_REL
    width = got.shape[-1] if got.ndim else 1
    row_rel = _normwise(got, ref, width) if got.size else np.zeros(1)
    blk_rel = head_rel = None
    if block is not None and got.size:
        assert width % block == 0, f"{what}: row width {width} is not a multiple of {block}"
        blk_rel = _normwise(got, ref, block)
        nh = width // block
        g3 = got.reshape(-1, nh, block).transpose(1, 0, 2).reshape(nh, -1)
        r3 = ref.reshape(-1, nh, block).transpose(1, 0, 2).reshape(nh, -1)
        head_rel = _normwise(g3, r3, g3.shape[1])
    stats = dict(what=what, dtype=dtype, elements=int(got.size), max_abs=float(err.max()) if got.size else 0.0,
                 max_row_rel=float(row_rel.max()),
                 max_head_rel=None if head_rel is None else float(head_rel.max()),
                 max_block_rel=None if blk_rel is None else float(blk_rel.max()),
                 ref_rms=float(np.sqrt(np.mean(ref * ref))) if got.size else 0.0)
    _report(stats)
    if bad.any():
        idx = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {err.size} elements beyond {bar}; "
                             f"max err {err.max():.4g} at {idx} (gpu {got[idx]:.6g}, oracle {ref[idx]:.6g})")
    if row_rel.max() > nbar:
        i = int(np.argmax(row_rel))
        raise AssertionError(f"{what}: row {i} normwise error {row_rel[i]:.3g} > {nbar} "
                             f"({int((row_rel > nbar).sum())} of {row_rel.size} rows)")
    if head_rel is not None and head_rel.max() > nbar:
        i = int(np.argmax(head_rel))
        raise AssertionError(f"{what}: head {i} normwise error over all rows {head_rel[i]:.3g} > {nbar}")
    if blk_rel is not None and blk_rel.max() > bbar:
        i = int(np.argmax(blk_rel))
        raise AssertionError(f"{what}: head block {i} (row {i * block // width}, head {i % (width // block)}) "
                             f"normwise error {blk_rel[i]:.3g} > {bbar} ({int((blk_rel > bbar).sum())} of "
                             f"{blk_rel.size} blocks)")
    return float(err.max()) if got.size else 0.0


def _report(stats: dict) -> None:
    import json
    import os
    print("PARITY " + json.dumps(stats), flush=True)
    path = os.environ.get("MLA_PARITY_LOG")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps(stats) + "\n")


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


# ---------------------------------------------------------------- gradients
GRAD_FROB_REL = 1e-2   # the whole tensor, normwise
GRAD_SLICE_REL = 2e-2  # every row / head slice, normwise
GRAD_FLOOR = 0.5       # slices below this fraction of a typical slice's norm count as near zero


def assert_tensor_close(got, ref, what: str, slices=(), frob_rel: float = GRAD_FROB_REL,
                        slice_rel: float = GRAD_SLICE_REL, floor: float = GRAD_FLOOR,
                        near_zero: dict | None = None) -> float:
    """Normwise comparison of a computed tensor (a gradient, a recurrent
    state) with the oracle's, as a whole and slice by slice.

    The whole tensor must satisfy ||gpu - oracle|| <= frob_rel ||oracle||.
    `slices` lists (label, shape, axes): the tensors are viewed with `shape`
    (None keeps theirs) and every index combination of `axes` is one slice
    (e.g. one token row, or one head).  With typ = rms * sqrt(n_s) the norm
    of a typical slice (rms of the whole tensor, n_s elements per slice):
      * a slice with ||oracle_s|| >= floor * typ must satisfy
        ||gpu_s - oracle_s|| <= slice_rel * ||oracle_s||;
      * a smaller one (its exact value is near zero, e.g. where a gradient
        is a small difference) ||gpu_s - oracle_s|| <= z * typ, with
        z = near_zero[label] if given, else slice_rel * floor.
    A wrong head, or a few wrong rows, of a large tensor fail here even when
    the whole-tensor error stays small.  Returns the whole-tensor relative
    error; every figure is printed."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    frob = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    stats = dict(what=what, elements=int(got.size), ref_rms=rms, frob_rel=frob)
    fails = []
    if frob > frob_rel:
        fails.append(f"relative Frobenius error {frob:.3g} > {frob_rel}")
    for label, shape, axes in slices:
        g = got.reshape(shape) if shape is not None else got
        r = ref.reshape(shape) if shape is not None else ref
        other = tuple(a for a in range(g.ndim) if a not in axes)
        n_s = int(np.prod([g.shape[a] for a in other])) if other else 1
        en = np.sqrt(np.sum((g - r) ** 2, axis=other)).ravel()
        rn = np.sqrt(np.sum(r * r, axis=other)).ravel()
        typ = rms * np.sqrt(n_s)
        z = (near_zero or {}).get(label, slice_rel * floor)
        small = rn < floor * typ
        bar = np.where(small, z * typ, slice_rel * rn)
        # errors in units of each slice's own bar
        ratio = en / np.where(bar > 0, bar, 1.0)
        stats[f"max_{label}_rel"] = float(np.max(np.where(small, 0.0, en / np.where(rn > 0, rn, 1.0))))
        stats[f"max_{label}_small_abs"] = float(np.max(np.where(small, en / max(typ, 1e-300), 0.0)))
        if ratio.max() > 1.0:
            i = int(np.argmax(ratio))
            idx = np.unravel_index(i, [g.shape[a] for a in axes])
            kind = (f"error {en[i] / max(typ, 1e-300):.3g} of a typical slice > {z}" if small[i]
                    else f"normwise error {en[i] / rn[i]:.3g} > {slice_rel}")
            fails.append(f"{label} {tuple(int(x) for x in idx)}: {kind} "
                         f"({int((ratio > 1).sum())} of {ratio.size} {label}s)")
    _report(stats)
    assert not fails, f"{what}: " + "; ".join(fails)
    return frob

"""Pins that tie the CPU oracle to something other than itself.

Each pin is a function ``pin_xxx(o)`` taking a loaded oracle build and raising
AssertionError when the oracle disagrees with what the pages or mathematics
fix.  The default build must pass all of them; every planted-mistake build
must fail at least one (see test_oracle_mutants.py).

Sources: page "Gated MLA（矩阵吸收版）" sections 矩阵吸收的核心思路 (absorption),
完整计算流（四步） (steps 2-4), 代码对照 (the forward listing) and the warning
box on associativity; page "符号表" sections MLA 变量 and Einsum 速查.
"""
from __future__ import annotations

import json
import os

import numpy as np

import datagen as dg

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f(d, k):
    return dg.as_f32(d[k])


def _args(d):
    return [_f(d, k) for k in ("q", "c", "w_uk", "w_uv", "gate")]


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.abs(a - b)
    bad = err > atol + rtol * np.abs(b)
    assert not bad.any(), f"{what}: max err {err.max():.3e} ({bad.sum()} elements out of tolerance)"


# ---------------------------------------------------------------- P1
def pin_absorbed_equals_decompressed(o):
    """Absorbed route equals decompressed K = c W_UK^T, V = c W_UV^T route
    (associativity; the importantbox and warningbox of the MLA page)."""
    for (B, T, H, dq, dv, r, scale, seed) in [(2, 9, 3, 4, 5, 7, 0.8, 11), (1, 17, 2, 3, 2, 6, 1.3, 12)]:
        d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.F32, seed=seed)
        a = o.prefill(*_args(d), scale)
        b = o.prefill_decompressed(*_args(d), scale)
        _close(a, b, 1e-12, 1e-14, "absorbed vs decompressed")


# ---------------------------------------------------------------- P2
def pin_attention_rows(o):
    """Causal softmax: each row sums to 1, keys after the query get weight 0,
    every visible key gets a positive weight."""
    d = dg.prefill_inputs(2, 7, 3, 4, 4, 5, dtype=dg.F32, seed=21)
    A = o.attn(_f(d, "q"), _f(d, "c"), _f(d, "w_uk"), 0.9)
    T = A.shape[-1]
    upper = np.triu(np.ones((T, T), dtype=bool), k=1)
    assert np.all(np.isfinite(A)), "attention weights not finite"
    assert np.all(A[..., upper] == 0.0), "weight on a future key"
    assert np.all(A[..., ~upper] > 0.0), "zero weight on a visible key"
    _close(A.sum(-1), np.ones(A.shape[:-1]), 1e-13, 0.0, "row sums")


# ---------------------------------------------------------------- P3
def pin_first_position_closed_form(o):
    """At t=0 only the query's own latent is visible, so the output is
    sigmoid(g) * (c_0 W_UV[h]^T), independent of q and of the scale."""
    B, T, H, dq, dv, r = 2, 5, 3, 4, 6, 8
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.F32, seed=31)
    c, w_uv, g = _f(d, "c").astype(np.float64), _f(d, "w_uv").astype(np.float64), _f(d, "gate").astype(np.float64)
    expect = np.einsum("bj,hvj->bhv", c[:, 0, :], w_uv).reshape(B, H * dv) * _sigmoid(g[:, 0, :])
    for scale in (0.5, 3.0):
        got = o.prefill(*_args(d), scale)[:, 0, :]
        _close(got, expect, 1e-13, 1e-15, f"t=0 closed form (scale={scale})")


# ---------------------------------------------------------------- P4
def pin_zero_scale_prefix_mean(o):
    """scale = 0 makes every visible key equally weighted, so the latent
    output is the prefix mean of c (a cumulative-sum closed form)."""
    B, T, H, dq, dv, r = 2, 11, 2, 3, 4, 5
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.F32, seed=41)
    c = _f(d, "c").astype(np.float64)
    w_uv, g = _f(d, "w_uv").astype(np.float64), _f(d, "gate").astype(np.float64)
    mean = np.cumsum(c, axis=1) / np.arange(1, T + 1)[None, :, None]
    expect = np.einsum("btj,hvj->bthv", mean, w_uv).reshape(B, T, H * dv) * _sigmoid(g)
    _close(o.prefill(*_args(d), 0.0), expect, 1e-12, 1e-15, "scale=0 prefix mean")


# ---------------------------------------------------------------- P5
def pin_reduces_to_sdpa(o):
    """With H=1, d_q=d_v=r, W_UK=W_UV=I and a saturated gate the layer is
    plain causal softmax attention with K=V=c; compare with PyTorch's
    scaled_dot_product_attention in float64 on the CPU.  A second case keeps
    general weights and feeds SDPA the decompressed K and V per head."""
    import torch
    import torch.nn.functional as F

    B, T, r = 2, 13, 6
    d = dg.prefill_inputs(B, T, 1, r, r, r, dtype=dg.F32, seed=51)
    eye = np.eye(r, dtype=np.float32)[None]
    gate = np.full((B, T, r), 40.0, dtype=np.float32)  # sigmoid(40) == 1.0 in float64
    q, c = _f(d, "q"), _f(d, "c")
    for scale in (0.37, 1.0, 2.5):
        got = o.prefill(q, c, eye, eye, gate, scale)
        qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)  # [B,1,T,r]
        ct_ = torch.from_numpy(c.astype(np.float64))[:, None]            # [B,1,T,r]
        ref = F.scaled_dot_product_attention(qt, ct_, ct_, is_causal=True, scale=scale)
        _close(got, ref[:, 0].numpy(), 1e-12, 1e-14, f"SDPA reduction (scale={scale})")

    B, T, H, dq, dv, r = 2, 10, 3, 4, 5, 7
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.F32, seed=52)
    q, c, wk, wv, g = [torch.from_numpy(x.astype(np.float64)) for x in _args(d)]
    K = torch.einsum("btj,hdj->bhtd", c, wk)
    V = torch.einsum("btj,hvj->bhtv", c, wv)
    ref = F.scaled_dot_product_attention(q.permute(0, 2, 1, 3), K, V, is_causal=True, scale=0.6)
    ref = ref.permute(0, 2, 1, 3).reshape(B, T, H * dv) * torch.sigmoid(g)
    _close(o.prefill(*_args(d), 0.6), ref.numpy(), 1e-12, 1e-14, "SDPA with decompressed K,V")


# ---------------------------------------------------------------- P6
def dense_forward(q, c, w_uk, w_uv, gate, scale):
    """Brute force on tiny shapes, written independently of the oracle: for
    each (batch, head) the whole T x T weight matrix is formed at once from
    the definition on page "Gated MLA（矩阵吸收版）", section 完整计算流（四步）
    (absorbed query times latent, keys after the query get weight zero, rows
    normalised), then applied to the latent and projected by W_UV; output
    columns h*d_v .. h*d_v + d_v - 1 of each row are gated by the sigmoid."""
    q, c, w_uk, w_uv, gate = [np.asarray(x, dtype=np.float64) for x in (q, c, w_uk, w_uv, gate)]
    B, T, H, _ = q.shape
    dv = w_uv.shape[1]
    allowed = np.arange(T)[None, :] <= np.arange(T)[:, None]  # [query, key]
    out = np.zeros((B, T, H * dv))
    for b in range(B):
        for h in range(H):
            logits = scale * ((q[b, :, h, :] @ w_uk[h]) @ c[b].T)
            top = np.where(allowed, logits, -np.inf).max(axis=1, keepdims=True)
            e = np.where(allowed, np.exp(np.where(allowed, logits - top, 0.0)), 0.0)
            weights = e / e.sum(axis=1, keepdims=True)
            o = (weights @ c[b]) @ w_uv[h].T  # [T, dv]
            cols = slice(h * dv, (h + 1) * dv)
            out[b, :, cols] = o / (1.0 + np.exp(-gate[b, :, cols]))
    return out


def pin_dense_brute_force(o):
    """Plain-loop oracle equals the dense per-(batch, head) brute force."""
    for (B, T, H, dq, dv, r, scale, seed) in [(2, 16, 3, 4, 2, 8, 0.7, 61), (1, 5, 2, 1, 3, 2, 1.9, 62),
                                              (2, 1, 1, 2, 2, 3, 1.0, 63)]:
        d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.F32, seed=seed)
        _close(o.prefill(*_args(d), scale), dense_forward(*_args(d), scale), 1e-12, 1e-14,
               f"dense brute force B{B} T{T} H{H}")


# ---------------------------------------------------------------- P7
def pin_decode_is_last_prefill_row(o):
    """Decode over a cache of len rows equals prefill row len-1: the cached
    latent already holds the new token's own c."""
    B, T, H, dq, dv, r = 3, 12, 2, 4, 3, 6
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.F32, seed=71)
    q, c, wk, wv, g = _args(d)
    lens = np.array([12, 1, 7], dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)])
    cache = np.concatenate([c[i, :lens[i]] for i in range(B)], axis=0)
    qd = np.stack([q[i, lens[i] - 1] for i in range(B)])
    gd = np.stack([g[i, lens[i] - 1] for i in range(B)])
    got = o.decode(qd, cache, cu, wk, wv, gd, 0.8)
    ref = o.prefill(q, c, wk, wv, g, 0.8, rows=[i * T + lens[i] - 1 for i in range(B)])
    _close(got, ref, 1e-13, 1e-15, "decode vs prefill last row")
    # decode of a subset of sequences picks the same rows
    sub = o.decode(qd, cache, cu, wk, wv, gd, 0.8, seqs=[2, 0])
    _close(sub, got[[2, 0]], 0.0, 0.0, "decode subset")


def pin_decode_closed_forms(o):
    """Decode alone: a one-row cache gives sigmoid(g) * (c W_UV[h]^T), and
    scale = 0 gives the mean of the whole cache, whatever q is."""
    H, dq, dv, r = 3, 4, 5, 6
    lens = np.array([1, 4, 1, 9], dtype=np.int64)
    d = dg.decode_inputs(4, H, dq, dv, r, dtype=dg.F32, seed=75, lengths=lens)
    cache = _f(d, "c_cache").astype(np.float64)
    wv, g = _f(d, "w_uv").astype(np.float64), _f(d, "gate").astype(np.float64)
    cu = d["cu_seqlens"].astype(np.int64)
    args = [_f(d, "q"), _f(d, "c_cache"), cu, _f(d, "w_uk"), _f(d, "w_uv"), _f(d, "gate")]
    got = o.decode(*args, 1.7)
    for i in (0, 2):
        expect = np.einsum("j,hvj->hv", cache[cu[i]], wv).reshape(-1) * _sigmoid(g[i])
        _close(got[i], expect, 1e-13, 1e-15, f"decode one-row cache seq {i}")
    got0 = o.decode(*args, 0.0)
    for i in range(4):
        mean = cache[cu[i]:cu[i + 1]].mean(axis=0)
        expect = np.einsum("j,hvj->hv", mean, wv).reshape(-1) * _sigmoid(g[i])
        _close(got0[i], expect, 1e-12, 1e-15, f"decode scale=0 mean seq {i}")


# ---------------------------------------------------------------- structure
def pin_causality_and_independence(o):
    """Row t depends on c only through positions <= t, and batches are
    independent: perturbing later positions or another batch leaves it."""
    B, T, H, dq, dv, r = 2, 9, 2, 3, 3, 4
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.F32, seed=81)
    q, c, wk, wv, g = _args(d)
    base = o.prefill(q, c, wk, wv, g, 1.1)
    c2 = c.copy()
    c2[0, 5:] += 1.0
    c2[1] *= -2.0
    pert = o.prefill(q, c2, wk, wv, g, 1.1)
    _close(pert[0, :5], base[0, :5], 0.0, 0.0, "causality")
    assert np.abs(pert[0, 5:] - base[0, 5:]).max() > 1e-3, "later rows ignore their keys"
    assert np.abs(pert[1] - base[1]).max() > 1e-3, "batch 1 ignores its keys"


def pin_head_permutation(o):
    """Permuting heads (q, W_UK, W_UV and gate blocks together) permutes the
    output's head blocks the same way."""
    B, T, H, dq, dv, r = 1, 6, 4, 3, 2, 5
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.F32, seed=91)
    q, c, wk, wv, g = _args(d)
    perm = np.array([2, 0, 3, 1])
    gp = g.reshape(B, T, H, dv)[:, :, perm].reshape(B, T, H * dv)
    a = o.prefill(q[:, :, perm], c, wk[perm], wv[perm], gp, 0.9)
    b = o.prefill(q, c, wk, wv, g, 0.9).reshape(B, T, H, dv)[:, :, perm].reshape(B, T, H * dv)
    _close(a, b, 0.0, 0.0, "head permutation")


# ---------------------------------------------------------------- golden
def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def pin_golden_worked_examples(o):
    """Hand-derived worked examples (see each fixture's derivation)."""
    names = sorted(n for n in os.listdir(GOLDEN) if n.startswith("worked_") and n.endswith(".json"))
    assert names, "no worked examples found"
    for n in names:
        g = load_golden(n)
        ins = {k: np.array(v, dtype=np.float32) for k, v in g["inputs"].items()}
        got = o.prefill(ins["q"], ins["c"], ins["w_uk"], ins["w_uv"], ins["gate"], float(g["scale"]))
        expect = np.array(g["expected"], dtype=np.float64)
        _close(got, expect, 1e-14, 1e-15, n)


# ---------------------------------------------------------------- chunked prefill
def dense_extend(q, c, w_uk, w_uv, gate, scale):
    """dense_forward for a chunk of T queries after a cached prefix: c holds
    S >= T rows per sequence and query t sits at position S - T + t."""
    q, c, w_uk, w_uv, gate = [np.asarray(x, dtype=np.float64) for x in (q, c, w_uk, w_uv, gate)]
    B, T, H, _ = q.shape
    S = c.shape[1]
    dv = w_uv.shape[1]
    allowed = np.arange(S)[None, :] <= (S - T + np.arange(T))[:, None]  # [query, key]
    out = np.zeros((B, T, H * dv))
    for b in range(B):
        for h in range(H):
            logits = scale * ((q[b, :, h, :] @ w_uk[h]) @ c[b].T)
            top = np.where(allowed, logits, -np.inf).max(axis=1, keepdims=True)
            e = np.where(allowed, np.exp(np.where(allowed, logits - top, 0.0)), 0.0)
            o = ((e / e.sum(axis=1, keepdims=True)) @ c[b]) @ w_uv[h].T
            cols = slice(h * dv, (h + 1) * dv)
            out[b, :, cols] = o / (1.0 + np.exp(-gate[b, :, cols]))
    return out


def pin_extend_matches_prefill_rows(o):
    """A chunk of the last T positions over the whole latent equals rows
    S-T .. S-1 of the prefill of the full sequence (T = S, 1 and between)."""
    B, S, H, dq, dv, r = 2, 23, 3, 4, 5, 6
    d = dg.prefill_inputs(B, S, H, dq, dv, r, dtype=dg.F32, seed=81)
    full = o.prefill(*_args(d), 0.9)
    q, c, wk, wv, g = _args(d)
    for T in (S, 1, 9):
        got = o.extend(q[:, S - T:], c, wk, wv, g[:, S - T:], 0.9)
        _close(got, full[:, S - T:], 1e-13, 1e-15, f"extend T={T} vs prefill rows")


def pin_extend_dense_brute_force(o):
    """Chunked prefill equals the dense brute force with the prefix mask."""
    for (B, T, S, H, dq, dv, r, scale, seed) in [(2, 5, 12, 2, 3, 4, 5, 0.7, 82), (1, 1, 7, 3, 2, 2, 4, 1.3, 83)]:
        d = dg.prefill_inputs(B, S, H, dq, dv, r, dtype=dg.F32, seed=seed)
        q, c, wk, wv, g = _args(d)
        got = o.extend(q[:, S - T:], c, wk, wv, g[:, S - T:], scale)
        _close(got, dense_extend(q[:, S - T:], c, wk, wv, g[:, S - T:], scale), 1e-12, 1e-14,
               f"extend dense brute force T={T} S={S}")


def pin_extend_one_query_is_decode(o):
    """A one-query chunk is a decode step: it equals the decode routine over
    the same latent laid out as a packed cache."""
    B, S, H, dq, dv, r = 3, 11, 2, 4, 3, 5
    d = dg.prefill_inputs(B, S, H, dq, dv, r, dtype=dg.F32, seed=84)
    q, c, wk, wv, g = _args(d)
    got = o.extend(q[:, S - 1:], c, wk, wv, g[:, S - 1:], 0.6)[:, 0]
    cu = np.arange(B + 1, dtype=np.int64) * S
    dec = o.decode(q[:, S - 1], c.reshape(B * S, r), cu, wk, wv, g[:, S - 1], 0.6)
    _close(got, dec, 1e-13, 1e-15, "extend T=1 vs decode")


ALL_PINS = [
    pin_absorbed_equals_decompressed,
    pin_attention_rows,
    pin_first_position_closed_form,
    pin_zero_scale_prefix_mean,
    pin_reduces_to_sdpa,
    pin_dense_brute_force,
    pin_decode_is_last_prefill_row,
    pin_decode_closed_forms,
    pin_causality_and_independence,
    pin_head_permutation,
    pin_golden_worked_examples,
    pin_extend_matches_prefill_rows,
    pin_extend_dense_brute_force,
    pin_extend_one_query_is_decode,
]

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


# ---------------------------------------------------------------- full layer
def _fwd(o, d, eps, scale, stage=0, **kw):
    return o.forward(*[dg.as_f32(d[k]) for k in dg.FORWARD_KEYS], eps, scale, stage=stage, **kw)


def pin_forward_closed_form_stages(o):
    """Selection matrices for the two down-projections make every stage of
    the full layer a closed form (page "Gated MLA（矩阵吸收版）", section 低秩压缩
    and section 完整计算流（四步） steps 1 and 4, eps = 0):
      * the latent input of a row is beta * s with beta > 0 and s_j = +-1, so
        its mean square is beta^2 and c = s * kv_norm exactly;
      * the query-latent input is alpha * e_k (one-hot), so the norm gives
        sign(alpha) sqrt(q_rank) e_k and q = sign(alpha) sqrt(q_rank)
        q_norm[k] * (column k of W_q_up);
      * W_gate = 0 gives sigmoid(0) = 1/2, and W_o = [I; 0] copies the gated
        core output into the first H*d_v outputs and zeroes the rest.
    The expected output is the (separately pinned) core on those closed
    forms."""
    rng = np.random.default_rng(41)
    B, T, H, dq, dv, r, q_rank = 2, 5, 2, 3, 2, 4, 6
    D, HV = q_rank + r + 3, H * dv
    k = rng.integers(0, q_rank, size=(B, T))
    alpha = rng.choice([-1.0, 1.0], size=(B, T)) * rng.uniform(0.5, 4.0, size=(B, T))
    beta = rng.uniform(0.5, 4.0, size=(B, T))
    sgn = rng.choice([-1.0, 1.0], size=(B, T, r))
    x = rng.standard_normal((B, T, D))
    x[..., :q_rank] = 0.0
    for b in range(B):
        for t in range(T):
            x[b, t, k[b, t]] = alpha[b, t]
    x[..., q_rank:q_rank + r] = beta[..., None] * sgn
    x = x.astype(np.float32)
    alpha = x[np.arange(B)[:, None], np.arange(T)[None, :], k].astype(np.float64)
    w_q_down = np.zeros((q_rank, D), np.float32)
    w_q_down[:, :q_rank] = np.eye(q_rank)
    w_kv_down = np.zeros((r, D), np.float32)
    w_kv_down[:, q_rank:q_rank + r] = np.eye(r)
    g_q = rng.uniform(0.5, 2.0, q_rank).astype(np.float32)
    g_kv = rng.uniform(0.5, 2.0, r).astype(np.float32)
    w_q_up = rng.standard_normal((H * dq, q_rank)).astype(np.float32)
    w_uk = (rng.standard_normal((H, dq, r)) / 2).astype(np.float32)
    w_uv = rng.standard_normal((H, dv, r)).astype(np.float32)
    w_gate = np.zeros((HV, D), np.float32)
    w_o = np.zeros((D, HV), np.float32)
    w_o[:HV] = np.eye(HV)
    scale = 0.45
    y, st = o.forward(x, w_kv_down, g_kv, w_q_down, g_q, w_q_up, w_uk, w_uv, w_gate, w_o, 0.0, scale,
                      stages=True)
    c_exp = sgn * g_kv.astype(np.float64)
    q_exp = (np.sign(alpha) * np.sqrt(q_rank) * g_q[k].astype(np.float64))[..., None] * \
        w_q_up.T[k].astype(np.float64)
    _close(st["c"].reshape(B, T, r), c_exp, 0.0, 0.0, "closed-form latent")
    _close(st["q"].reshape(B, T, H * dq), q_exp, 2e-7, 1e-12, "closed-form query")
    core = o.prefill(q_exp.reshape(B, T, H, dq), c_exp, w_uk, w_uv, np.zeros((B, T, HV)), scale)
    y_exp = np.concatenate([core, np.zeros((B, T, D - HV))], axis=-1)
    _close(y, y_exp, 2e-6, 1e-9, "closed-form full layer")


def pin_forward_norm_scale_invariance(o):
    """With eps = 0 an RMSNorm output does not change when its input is
    scaled, so scaling W_kv_down or W_q_down by a power of two leaves the
    layer's output bit-identical; q is linear in W_q_up, so doubling W_q_up
    and halving the softmax scale does too (page "Gated MLA（矩阵吸收版）",
    section 低秩压缩 and section 完整计算流（四步） steps 1-2)."""
    d = dg.forward_inputs(2, 7, 64, 32, 3, 4, 5, 8, dtype=dg.F32, seed=71)
    base = _fwd(o, d, 0.0, 0.6)
    for key, f, sc in (("w_kv_down", 4.0, 0.6), ("w_q_down", 0.25, 0.6), ("w_q_up", 2.0, 0.3)):
        e = dict(d)
        e[key] = dg.as_f32(d[key]) * np.float32(f)
        _close(_fwd(o, e, 0.0, sc), base, 1e-13, 1e-15, f"{key} scaled by {f}")


def _brute_forward(d, eps, scale, f64=False):
    """The whole layer in plain Python loops on float64 scalars, attention
    by the decompressed route (k = W_UK[h] c_u, v = W_UV[h] c_u per key),
    written from page "Gated MLA（矩阵吸收版）": section 低秩压缩 (c), section
    矩阵吸收的核心思路 (the standard route), section 完整计算流（四步） steps 1-4."""
    import math
    # f64: take the values as float64 (finite differences), else as float32
    f = {k: (np.asarray(d[k], np.float64) if f64 else dg.as_f32(d[k]).astype(np.float64)).tolist()
         for k in dg.FORWARD_KEYS}
    B, T, D, q_rank, H, dq, dv, r = (d[k] for k in ("B", "T", "D", "q_rank", "H", "d_q", "d_v", "r"))

    def lin(vec, W):
        return [sum(a * b for a, b in zip(vec, row)) for row in W]

    def norm(vec, gain):
        ms = sum(v * v for v in vec) / len(vec)
        return [v / math.sqrt(ms + eps) * g for v, g in zip(vec, gain)]

    y = np.zeros((B, T, D))
    for b in range(B):
        xs = f["x"][b]
        c = [norm(lin(xs[u], f["w_kv_down"]), f["kv_norm"]) for u in range(T)]
        for t in range(T):
            qv = lin(norm(lin(xs[t], f["w_q_down"]), f["q_norm"]), f["w_q_up"])
            gl = lin(xs[t], f["w_gate"])
            gated = []
            for h in range(H):
                qh = qv[h * dq:(h + 1) * dq]
                keys = [lin(c[u], f["w_uk"][h]) for u in range(t + 1)]
                vals = [lin(c[u], f["w_uv"][h]) for u in range(t + 1)]
                sc = [scale * sum(a * b for a, b in zip(qh, kk)) for kk in keys]
                m = max(sc)
                w = [math.exp(s_ - m) for s_ in sc]
                z = sum(w)
                for v in range(dv):
                    ov = sum(w[u] * vals[u][v] for u in range(t + 1)) / z
                    gated.append(ov / (1.0 + math.exp(-gl[h * dv + v])))
            y[b, t] = lin(gated, f["w_o"])
    return y


def pin_forward_brute_force(o):
    """The full layer equals a plain-loop brute force that takes the
    decompressed route, with eps > 0 (float32 storage of the stage
    results accounts for the tolerance)."""
    for (B, T, D, q_rank, H, dq, dv, r, eps, scale, seed) in [(1, 4, 6, 4, 2, 2, 3, 5, 1e-3, 0.7, 81),
                                                               (2, 3, 5, 3, 1, 3, 2, 4, 0.05, 1.3, 82)]:
        d = dg.forward_inputs(B, T, D, q_rank, H, dq, dv, r, dtype=dg.F32, seed=seed)
        _close(_fwd(o, d, eps, scale), _brute_forward(d, eps, scale), 2e-6, 1e-7,
               f"full-layer brute force B{B} T{T} D{D}")


def pin_round_bf16(o):
    """The oracle's bf16 rounding (nearest, ties to even, from the float64
    value) against fixed cases and two other implementations on float32
    inputs (the bit-pattern rounding of the data generator and torch's
    float32 -> bfloat16 conversion)."""
    import torch
    one = 1.0
    u = 2.0 ** -8  # half a bf16 ulp at 1
    cases = [(one + u, one), (one + 3 * u, one + 4 * u), (-(one + u), -one), (one + u + 2.0 ** -40, one + 2 * u),
             (one + 0.99 * u, one), (0.0, 0.0), (1.5 * 2.0 ** -133, 2.0 * 2.0 ** -133),
             (2.5 * 2.0 ** -133, 2.0 * 2.0 ** -133), (3.3895313892515355e38 + 2.0 ** 118, 3.3895313892515355e38),
             (3.3895313892515355e38 + 2.0 ** 119, np.inf), (-7.0, -7.0), (1.0 / 3.0, 0.333984375)]
    got = o.round_bf16(np.array([a for a, _ in cases]))
    for (a, want), g in zip(cases, got):
        assert g == want, f"round_bf16({a!r}) = {g!r}, expected {want!r}"
    rng = np.random.default_rng(91)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-60, 60, 20000))).astype(np.float32)
    v = np.concatenate([v, dg.bf16_bits_to_f32(rng.integers(0, 0x7F7F, 2000).astype(np.uint16)) *
                        np.float32(1.0 + 2.0 ** -8)])
    ref_bits = dg.bf16_bits_to_f32(dg.f32_to_bf16_bits(v)).astype(np.float64)
    ref_torch = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = o.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, ref_bits), "round_bf16 differs from the bit-pattern rounding"
    assert np.array_equal(got, ref_torch), "round_bf16 differs from torch's bfloat16 conversion"


# ---------------------------------------------------------------- paged cache
def _paged_case(seed, B, H, dq, dv, r, lens, page_size):
    d = dg.decode_inputs(B, H, dq, dv, r, dtype=dg.F32, seed=seed, lengths=lens)
    lay = dg.paged_layout(d["lengths"], page_size, seed=seed)
    pool = dg.scatter_to_pages(d["c_cache"], d["cu_seqlens"], lay)
    return d, lay, pool


def pin_paged_decode_matches_packed(o):
    """A paged cache holds the same rows as the packed one (the pages cache
    only c; paging is storage): decode over shuffled pages, with NaN in every
    slot no sequence owns, equals decode over the packed rows exactly."""
    for (seed, B, H, dq, dv, r, lens, ps) in [(101, 4, 3, 4, 3, 8, [1, 9, 32, 70], 8),
                                              (102, 3, 2, 2, 2, 5, [64, 5, 33], 32)]:
        d, lay, pool = _paged_case(seed, B, H, dq, dv, r, lens, ps)
        f = dg.as_f32
        got = o.decode_paged(f(d["q"]), pool, lay["block_table"], d["lengths"], f(d["w_uk"]), f(d["w_uv"]),
                             f(d["gate"]), 0.8)
        ref = o.decode(f(d["q"]), f(d["c_cache"]), d["cu_seqlens"].astype(np.int64), f(d["w_uk"]),
                       f(d["w_uv"]), f(d["gate"]), 0.8)
        _close(got, ref, 0.0, 0.0, f"paged decode page_size {ps}")


def pin_paged_extend_matches_packed(o):
    """Chunked prefill over shuffled pages equals chunked prefill over the
    contiguous latent."""
    B, S, T, H, dq, dv, r, ps = 2, 21, 6, 2, 3, 2, 5, 8
    d = dg.prefill_inputs(B, S, H, dq, dv, r, dtype=dg.F32, seed=103)
    f = dg.as_f32
    lay = dg.paged_layout([S] * B, ps, seed=103)
    cu = np.arange(B + 1) * S
    pool = dg.scatter_to_pages(f(d["c"]).reshape(B * S, r), cu, lay)
    got = o.extend_paged(f(d["q"])[:, S - T:], pool, lay["block_table"], S, f(d["w_uk"]), f(d["w_uv"]),
                         f(d["gate"])[:, S - T:], 0.7)
    ref = o.extend(f(d["q"])[:, S - T:], f(d["c"]), f(d["w_uk"]), f(d["w_uv"]), f(d["gate"])[:, S - T:], 0.7)
    _close(got, ref, 0.0, 0.0, "paged extend")


def pin_cache_append_then_decode(o):
    """Appending each sequence's new latent at position len_i and decoding
    over len_i + 1 rows equals decoding over the packed rows with the new row
    at the end of each sequence; no other slot of the pool changes."""
    B, H, dq, dv, r, ps = 3, 2, 3, 2, 6, 8
    lens = np.array([7, 8, 20])
    full = dg.decode_inputs(B, H, dq, dv, r, dtype=dg.F32, seed=104, lengths=lens + 1)
    f = dg.as_f32
    cu_full = full["cu_seqlens"].astype(np.int64)
    new_rows = f(full["c_cache"])[cu_full[1:] - 1]
    keep = np.ones(cu_full[-1], bool)
    keep[cu_full[1:] - 1] = False
    old = f(full["c_cache"])[keep]
    cu_old = np.concatenate([[0], np.cumsum(lens)])
    lay = dg.paged_layout(lens + 1, ps, seed=104)
    pool = dg.scatter_to_pages(old, cu_old, lay)
    after = o.cache_append(new_rows, pool, lay["block_table"], lens)
    changed = ~np.all((after == pool) | (np.isnan(after) & np.isnan(pool)), axis=-1)
    assert changed.sum() == B, f"append changed {changed.sum()} slots, expected {B}"
    got = o.decode_paged(f(full["q"]), after, lay["block_table"], lens + 1, f(full["w_uk"]), f(full["w_uv"]),
                         f(full["gate"]), 0.9)
    ref = o.decode(f(full["q"]), f(full["c_cache"]), cu_full, f(full["w_uk"]), f(full["w_uv"]), f(full["gate"]), 0.9)
    _close(got, ref, 0.0, 0.0, "append then paged decode")


# ---------------------------------------------------------------- backward
def pin_backward_finite_differences(o):
    """Every element of every gradient of the core against a central finite
    difference of the loss sum(dout * out), the forward evaluated by the
    independent float64 brute force above (dense_forward): calculus, not
    the oracle's own arithmetic.  Two tiny shapes, scales 0.7 and 1.6."""
    for (B, T, H, dq, dv, r, scale, seed) in [(2, 5, 2, 3, 2, 4, 0.7, 111), (1, 4, 3, 2, 3, 5, 1.6, 112)]:
        d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.F32, seed=seed)
        args = {k: _f(d, k).astype(np.float64) for k in ("q", "c", "w_uk", "w_uv", "gate")}
        dout = np.random.default_rng(seed).standard_normal((B, T, H * dv))
        g = o.prefill_backward(*[args[k] for k in ("q", "c", "w_uk", "w_uv", "gate")],
                               dout.astype(np.float32), scale)
        dout64 = dout.astype(np.float32).astype(np.float64)

        def loss(a):
            return float(np.sum(dout64 * dense_forward(a["q"], a["c"], a["w_uk"], a["w_uv"], a["gate"], scale)))

        eps = 1e-6
        for key, gk in (("q", "dq"), ("c", "dc"), ("w_uk", "dw_uk"), ("w_uv", "dw_uv"), ("gate", "dgate")):
            x = args[key]
            fd = np.empty(x.size)
            for i in range(x.size):
                orig = x.flat[i]
                x.flat[i] = orig + eps
                lp = loss(args)
                x.flat[i] = orig - eps
                lm = loss(args)
                x.flat[i] = orig
                fd[i] = (lp - lm) / (2 * eps)
            got = g[gk].reshape(-1)
            _close(got, fd, 1e-6, 1e-8, f"d{key} vs finite differences (B{B} T{T} H{H})")


def pin_backward_special_cases(o):
    """Closed forms: with scale 0 the scores carry no gradient, so dq and
    dW_UK vanish exactly; at T = 1 the softmax is the constant 1, so
    dc_0 = sum_h W_UV[h]^T (dout_h * sigmoid(g_h)) and dq vanishes."""
    B, T, H, dq, dv, r = 2, 6, 3, 4, 2, 5
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.F32, seed=113)
    dout = np.random.default_rng(113).standard_normal((B, T, H * dv)).astype(np.float32)
    g = o.prefill_backward(*_args(d), dout, 0.0)
    assert np.all(g["dq"] == 0.0) and np.all(g["dw_uk"] == 0.0), "scale 0: query gradients must vanish"
    d1 = dg.prefill_inputs(B, 1, H, dq, dv, r, dtype=dg.F32, seed=114)
    dout1 = np.random.default_rng(114).standard_normal((B, 1, H * dv)).astype(np.float32)
    g1 = o.prefill_backward(*_args(d1), dout1, 0.9)
    wv = _f(d1, "w_uv").astype(np.float64)
    s = _sigmoid(_f(d1, "gate").astype(np.float64)).reshape(B, H, dv)
    want = np.einsum("hvj,bhv->bj", wv, dout1.astype(np.float64).reshape(B, H, dv) * s)
    _close(g1["dc"][:, 0], want, 1e-12, 1e-14, "T=1 dc closed form")
    _close(g1["dq"], np.zeros_like(g1["dq"]), 0.0, 1e-14, "T=1 dq")


def pin_lse_matches_library(o):
    """The log-sum-exp of each causal score row equals scipy's logsumexp of
    the scores formed densely in numpy (a library routine)."""
    from scipy.special import logsumexp
    B, T, H, dq, dv, r, scale = 2, 7, 3, 4, 2, 5, 0.8
    d = dg.prefill_inputs(B, T, H, dq, dv, r, dtype=dg.F32, seed=115)
    q, c, wk = (_f(d, k).astype(np.float64) for k in ("q", "c", "w_uk"))
    want = np.empty((B, H, T))
    for b in range(B):
        for h in range(H):
            sc = scale * (q[b, :, h, :] @ wk[h]) @ c[b].T
            for t in range(T):
                want[b, h, t] = logsumexp(sc[t, :t + 1])
    _close(o.prefill_lse(_f(d, "q"), _f(d, "c"), _f(d, "w_uk"), scale), want, 1e-13, 1e-13, "lse")


def pin_varlen_mixed_batch(o):
    """A varlen batch mixing a full prefill (S = T), a chunk after a cached
    prefix, a decode step (T = 1) and an empty chunk over one shuffled page
    pool equals, sequence by sequence, the separately written prefill and
    decode routines (and chunked prefill, itself pinned against both)."""
    H, dq, dv, r, ps = 2, 3, 2, 5, 8
    S = [13, 20, 9, 6]
    T = [13, 7, 1, 0]
    parts = [dg.prefill_inputs(1, s_, H, dq, dv, r, dtype=dg.F32, seed=120 + i) for i, s_ in enumerate(S)]
    f = dg.as_f32
    c_rows = np.concatenate([f(p["c"])[0] for p in parts])
    cu_k = np.concatenate([[0], np.cumsum(S)])
    lay = dg.paged_layout(S, ps, seed=120)
    pool = dg.scatter_to_pages(c_rows, cu_k, lay)
    q = np.concatenate([f(p["q"])[0, s_ - t_:] for p, s_, t_ in zip(parts, S, T)])
    g = np.concatenate([f(p["gate"])[0, s_ - t_:] for p, s_, t_ in zip(parts, S, T)])
    cu_q = np.concatenate([[0], np.cumsum(T)])
    wk, wv = f(parts[0]["w_uk"]), f(parts[0]["w_uv"])
    got = o.extend_varlen_paged(q, pool, lay["block_table"], cu_q, S, wk, wv, g, 0.6)
    full = o.prefill(f(parts[0]["q"]), f(parts[0]["c"]), wk, wv, f(parts[0]["gate"]), 0.6)[0]
    _close(got[cu_q[0]:cu_q[1]], full, 1e-13, 1e-15, "varlen prefill sequence")
    part1 = o.extend(f(parts[1]["q"])[:, S[1] - T[1]:], f(parts[1]["c"]), wk, wv, f(parts[1]["gate"])[:, S[1] - T[1]:],
                     0.6)[0]
    _close(got[cu_q[1]:cu_q[2]], part1, 1e-13, 1e-15, "varlen chunk after a prefix")
    dec = o.decode(f(parts[2]["q"])[:, S[2] - 1], f(parts[2]["c"])[0], np.array([0, S[2]]), wk, wv,
                   f(parts[2]["gate"])[:, S[2] - 1], 0.6)
    _close(got[cu_q[2]:cu_q[3]], dec, 1e-13, 1e-15, "varlen decode step")


def pin_layer_backward_finite_differences(o):
    """Every element of every gradient of the full layer (dx and the ten
    parameter tensors) against a central finite difference of sum(dy * y),
    y from the plain-loop float64 brute force of the layer above
    (_brute_forward, decompressed attention route), with eps > 0.  The
    oracle stores the forward's stage results as float32, which the
    tolerance covers."""
    B, T, D, q_rank, H, dq, dv, r, eps, scale = 1, 3, 6, 4, 2, 2, 3, 5, 1e-2, 0.7
    d = dg.forward_inputs(B, T, D, q_rank, H, dq, dv, r, dtype=dg.F32, seed=131)
    dy = np.random.default_rng(131).standard_normal((B, T, D)).astype(np.float32)
    g = o.forward_backward(*[dg.as_f32(d[k]) for k in dg.FORWARD_KEYS], dy, eps, scale)
    base = {k: dg.as_f32(d[k]).astype(np.float64) for k in dg.FORWARD_KEYS}
    dy64 = dy.astype(np.float64)

    def loss(p):
        e = dict(d)
        e.update(p)
        return float(np.sum(dy64 * _brute_forward(e, eps, scale, f64=True)))

    step = 1e-5
    names = dict(x="dx", w_kv_down="dw_kv_down", kv_norm="dkv_norm", w_q_down="dw_q_down", q_norm="dq_norm",
                 w_q_up="dw_q_up", w_uk="dw_uk", w_uv="dw_uv", w_gate="dw_gate", w_o="dw_o")
    for key, gk in names.items():
        xv = base[key]
        fd = np.empty(xv.size)
        for i in range(xv.size):
            orig = xv.flat[i]
            xv.flat[i] = orig + step
            lp = loss(base)
            xv.flat[i] = orig - step
            lm = loss(base)
            xv.flat[i] = orig
            fd[i] = (lp - lm) / (2 * step)
        _close(g[gk].reshape(-1), fd, 2e-5, 2e-6, f"{gk} vs finite differences")


# ----------------------------------------------------------------- chunk_kda
def _kda_arrays(d, s0=True):
    f = lambda x: dg.as_f32(x).astype(np.float64)
    return (f(d["q"]), f(d["k"]), f(d["v"]), np.asarray(d["g"], np.float64), np.asarray(d["beta"], np.float64),
            (np.asarray(d["s0"], np.float64) if (s0 and d["s0"] is not None) else None))


def _kda_global_solve(q, k, v, g, beta, s0, G):
    """The recurrence of chunk_kda unrolled over the whole sequence as one
    block (numpy, float64).  With Gam_t = sum_{u<=t} g_u per key channel and
    a_u = beta_u k_u, the state after step t is
      S_t = e^{Gam_t} * S0 + sum_{u<=t} (a_u * e^{Gam_t - Gam_u}) r_u^T,
    so the residuals r_t = v_t - k_t^T S_dec,t solve the unit lower-triangular
    system (I + A) R = V - (K * e^Gam) S0 with A_tu = sum_c k_t[c] a_u[c]
    e^{Gam_t[c] - Gam_u[c]} for u < t; then O = (Q * e^Gam) S0 + Bm R with
    Bm_tu of the same form with q_t, for u <= t.  Written from that
    derivation, independent of the step-by-step loop."""
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    o = np.zeros((B, T, HV, V))
    st = np.zeros((B, HV, K, V))
    for b in range(B):
        for hv in range(HV):
            h = hv // G
            qs, ks, vs, gs, bs = q[b, :, h], k[b, :, h], v[b, :, hv], g[b, :, hv], beta[b, :, hv]
            S0 = s0[b, hv] if s0 is not None else np.zeros((K, V))
            Gam = np.cumsum(gs, axis=0)                          # [T, K]
            a = bs[:, None] * ks                                  # [T, K]
            E = np.exp(Gam[:, None, :] - Gam[None, :, :])         # [t, u, K], e^{Gam_t - Gam_u}
            A = np.einsum("tc,uc,tuc->tu", ks, a, E) * np.tril(np.ones((T, T)), -1)
            Bm = np.einsum("tc,uc,tuc->tu", qs, a, E) * np.tril(np.ones((T, T)), 0)
            R = np.linalg.solve(np.eye(T) + A, vs - (ks * np.exp(Gam)) @ S0)
            o[b, :, hv] = (qs * np.exp(Gam)) @ S0 + Bm @ R
            st[b, hv] = np.exp(Gam[-1])[:, None] * S0 + (a * np.exp(Gam[-1] - Gam)).T @ R
    return o, st


def pin_kda_global_solve(o):
    """The oracle's step-by-step recurrence equals the one-block triangular
    solve above (GVA with G = 2, K != V, an initial state, ragged T)."""
    d = dg.kda_inputs(2, 37, 2, 2, 8, 6, dtype=dg.F32, seed=41, init_state=True)
    q, k, v, g, beta, s0 = _kda_arrays(d)
    got_o, got_s = o.kda(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], G=2)
    want_o, want_s = _kda_global_solve(q, k, v, g, beta, s0, 2)
    _close(got_o, want_o, 1e-10, 1e-12, "kda o vs the global solve")
    _close(got_s, want_s, 1e-10, 1e-12, "kda final state vs the global solve")


def pin_kda_overwrite_memory(o):
    """No decay (g = 0), full write strength (beta = 1) and one-hot keys: the
    delta rule overwrites row idx_t of the state with v_t, so after step t
    the state is S0 with each written row replaced by its latest value, and
    o_t = q_t^T of that table (a dictionary walk, not the recurrence)."""
    B, T, H, K, V = 1, 24, 1, 6, 4
    rng = np.random.default_rng(43)
    idx = rng.integers(0, K, size=T)
    kk = np.zeros((B, T, H, K), np.float32)
    kk[0, np.arange(T), 0, idx] = 1.0
    q = rng.standard_normal((B, T, H, K)).astype(np.float32)
    v = rng.standard_normal((B, T, H, V)).astype(np.float32)
    s0 = rng.standard_normal((B, H, K, V)).astype(np.float32)
    g = np.zeros((B, T, H, K), np.float32)
    beta = np.ones((B, T, H), np.float32)
    got, st = o.kda(q, kk, v, g, beta, s0)
    table = s0[0, 0].astype(np.float64).copy()
    for t in range(T):
        table[idx[t]] = v[0, t, 0]
        _close(got[0, t, 0], q[0, t, 0].astype(np.float64) @ table, 1e-12, 1e-12, f"overwrite o_{t}")
    _close(st[0, 0], table, 1e-12, 1e-12, "overwrite final state")


def pin_kda_decay_only(o):
    """beta = 0: nothing is written, the state is S0 decayed per key channel:
    o_t = sum_c q_t[c] e^{Gam_t[c]} S0[c, :] and S_T = e^{Gam_T} * S0."""
    d = dg.kda_inputs(1, 19, 3, 1, 5, 7, dtype=dg.F32, seed=47, init_state=True)
    d["beta"] = np.zeros_like(d["beta"])
    q, k, v, g, beta, s0 = _kda_arrays(d)
    got_o, got_s = o.kda(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])
    Gam = np.cumsum(g, axis=1)                                   # [B, T, HV, K]
    want_o = np.einsum("bthc,bthc,bhcv->bthv", q, np.exp(Gam), s0)
    _close(got_o, want_o, 1e-12, 1e-14, "decay-only o")
    _close(got_s, np.exp(Gam[:, -1])[..., None] * s0, 1e-12, 1e-14, "decay-only state")


def pin_kda_state_passing(o):
    """Running T1 positions, then the next T2 from the returned state, equals
    one run over T1 + T2 (the state is the whole carry between chunks)."""
    d = dg.kda_inputs(2, 30, 2, 2, 8, 8, dtype=dg.F32, seed=53, init_state=True)
    T1 = 13
    full_o, full_s = o.kda(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], G=2)
    cut = lambda x, a, b: np.ascontiguousarray(x[:, a:b])
    o1, s1 = o.kda(cut(d["q"], 0, T1), cut(d["k"], 0, T1), cut(d["v"], 0, T1), cut(d["g"], 0, T1),
                   cut(d["beta"], 0, T1), d["s0"], G=2)
    o2, s2 = o.kda(cut(d["q"], T1, 30), cut(d["k"], T1, 30), cut(d["v"], T1, 30), cut(d["g"], T1, 30),
                   cut(d["beta"], T1, 30), s1.astype(np.float32), G=2)
    # the carried state passes through float32 at the cut: compare at float32 precision
    _close(np.concatenate([o1, o2], axis=1), full_o, 1e-5, 1e-6, "state passing o")
    _close(s2, full_s, 1e-5, 1e-6, "state passing final state")


def pin_kda_gva_and_linearity(o):
    """GVA: G = 2 value heads per query/key head equals G = 1 with q and k
    repeated per value head.  Linearity: doubling v and S0 doubles o and the
    final state exactly (every step is linear in them)."""
    d = dg.kda_inputs(1, 21, 2, 2, 6, 5, dtype=dg.F32, seed=59, init_state=True)
    o2, s2 = o.kda(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], G=2)
    rep = lambda x: np.ascontiguousarray(np.repeat(x, 2, axis=2))
    o1, s1 = o.kda(rep(d["q"]), rep(d["k"]), d["v"], d["g"], d["beta"], d["s0"], G=1)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2), "GVA expansion differs"
    od, sd = o.kda(d["q"], d["k"], d["v"] * 2, d["g"], d["beta"], d["s0"] * 2, G=2)
    assert np.array_equal(od, 2 * o2) and np.array_equal(sd, 2 * s2), "not linear in (v, S0)"


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
    pin_forward_closed_form_stages,
    pin_forward_norm_scale_invariance,
    pin_forward_brute_force,
    pin_round_bf16,
    pin_paged_decode_matches_packed,
    pin_paged_extend_matches_packed,
    pin_cache_append_then_decode,
    pin_backward_finite_differences,
    pin_backward_special_cases,
    pin_lse_matches_library,
    pin_varlen_mixed_batch,
    pin_layer_backward_finite_differences,
    pin_kda_global_solve,
    pin_kda_overwrite_memory,
    pin_kda_decay_only,
    pin_kda_state_passing,
    pin_kda_gva_and_linearity,
]
